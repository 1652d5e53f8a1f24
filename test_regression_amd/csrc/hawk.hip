// hawk.hip -- the recurrence of the Hawk layer of the Hawk-Mesa hybrid (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section
// "Arquitetura (MesaNet)", bullet "Variante Hibrida": the hybrid model
// alternates LRU (Hawk) layers with Mesa layers.  The page names the layer
// only; the recurrence here is Hawk's published real-gated linear recurrent
// unit, per channel d with gate pre-activations ga, gx:
//   r_t = sigmoid(ga_t),  i_t = sigmoid(gx_t),  log a_t = -c softplus(-lam_d) r_t
//   h_t = a_t h_{t-1} + sqrt(1 - a_t^2) i_t x_t
// (1 - a^2 = 1 - e^{2 log a} is evaluated without cancellation for a near 1).
//
// It is HBM-bound and sequential in t, so it runs as a two-pass chunked
// scan that keeps every channel's chunks busy at once: pass 1 reduces each
// (sequence, chunk, channel) to its decay product P_c and its end state s_c
// from zero; pass 2 folds the earlier chunks' (P, s) into the chunk's start
// state and rescans the chunk, writing h.  A thread owns one channel of one
// chunk; consecutive threads take consecutive channels, so every load and
// store of a wave is one contiguous row piece.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

constexpr int kHawkUnroll = 8;

__device__ __forceinline__ float hawk_softplus(float z) { return z > 20.f ? z : log1pf(__expf(z)); }
__device__ __forceinline__ float hawk_sigmoid(float z) { return 1.0f / (1.0f + __expf(-z)); }

// One step's decay (as its log and value) and input term.  1 - a^2 is the
// short Taylor series of 1 - e^{2 log a} where the subtraction would cancel
// (2 log a > -1/16: the first dropped term is below 2^-24 relative), and
// 1 - a*a elsewhere (a < 0.97, so 1 - a*a > 0.06 keeps ~23 bits).
template <typename In>
__device__ __forceinline__ void hawk_step(In xv, In gav, In gxv, float csp, float& loga, float& a, float& u) {
    const float r = hawk_sigmoid(to_f32(gav));
    const float i = hawk_sigmoid(to_f32(gxv));
    loga = -csp * r;
    a = __expf(loga);
    const float z = 2.0f * loga;
    const float taylor = -z * (1.f + z * (0.5f + z * (1.f / 6.f + z * (1.f / 24.f + z * (1.f / 120.f)))));
    const float oma = z > -0.0625f ? taylor : 1.f - a * a;
    u = sqrtf(oma) * (i * to_f32(xv));
}

template <typename In>
__global__ __launch_bounds__(256) void hawk_summary_kernel(const In* __restrict__ x, const In* __restrict__ ga,
                                                           const In* __restrict__ gx, const float* __restrict__ lam,
                                                           float c, int T, int D, int d0, int Dn, int nc,
                                                           long n_threads, float* __restrict__ Plog,
                                                           float* __restrict__ S) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= n_threads) return;
    const int d = d0 + (int)(g % Dn);
    const long rem = g / Dn;
    const int ch = (int)(rem % nc);
    const long b = rem / nc;
    const int t0 = ch * kHawkChunk, t1 = min(T, t0 + kHawkChunk);
    const float csp = c * hawk_softplus(-lam[d]);
    float h = 0.f, lsum = 0.f;
    size_t i = ((size_t)b * T + t0) * D + d;
    int t = t0;
    for (; t + kHawkUnroll <= t1; t += kHawkUnroll) {
        In xr[kHawkUnroll], ar[kHawkUnroll], gr[kHawkUnroll];
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            xr[u] = x[i + (size_t)u * D];
            ar[u] = ga[i + (size_t)u * D];
            gr[u] = gx[i + (size_t)u * D];
        }
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            float la, av, v;
            hawk_step(xr[u], ar[u], gr[u], csp, la, av, v);
            h = av * h + v;
            lsum += la;
        }
        i += (size_t)kHawkUnroll * D;
    }
    for (; t < t1; ++t, i += D) {
        float la, av, v;
        hawk_step(x[i], ga[i], gx[i], csp, la, av, v);
        h = av * h + v;
        lsum += la;
    }
    const size_t j = ((size_t)b * nc + ch) * D + d;
    Plog[j] = lsum;   // log of the chunk's decay product
    S[j] = h;         // the chunk's end state from zero
}

template <typename In>
__global__ __launch_bounds__(256) void hawk_scan_kernel(const In* __restrict__ x, const In* __restrict__ ga,
                                                        const In* __restrict__ gx, const float* __restrict__ lam,
                                                        float c, const float* __restrict__ h0, int T, int D, int d0,
                                                        int Dn, int nc, long n_threads,
                                                        const float* __restrict__ Plog, const float* __restrict__ S,
                                                        float* __restrict__ y, float* __restrict__ h_final) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= n_threads) return;
    const int d = d0 + (int)(g % Dn);
    const long rem = g / Dn;
    const int ch = (int)(rem % nc);
    const long b = rem / nc;
    const int t0 = ch * kHawkChunk, t1 = min(T, t0 + kHawkChunk);
    const float csp = c * hawk_softplus(-lam[d]);
    // the chunk's start state: fold the earlier chunks' (P, s) in order,
    // eight summaries requested at a time
    float h = h0 ? h0[b * D + d] : 0.f;
    {
        const size_t j0 = (size_t)b * nc * D + d;
        int cc = 0;
        for (; cc + 8 <= ch; cc += 8) {
            float pl[8], sv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                pl[u] = Plog[j0 + (size_t)(cc + u) * D];
                sv[u] = S[j0 + (size_t)(cc + u) * D];
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) h = __expf(pl[u]) * h + sv[u];
        }
        for (; cc < ch; ++cc) h = __expf(Plog[j0 + (size_t)cc * D]) * h + S[j0 + (size_t)cc * D];
    }
    size_t i = ((size_t)b * T + t0) * D + d;
    int t = t0;
    for (; t + kHawkUnroll <= t1; t += kHawkUnroll) {
        In xr[kHawkUnroll], ar[kHawkUnroll], gr[kHawkUnroll];
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            xr[u] = x[i + (size_t)u * D];
            ar[u] = ga[i + (size_t)u * D];
            gr[u] = gx[i + (size_t)u * D];
        }
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            float la, av, v;
            hawk_step(xr[u], ar[u], gr[u], csp, la, av, v);
            h = av * h + v;
            y[i + (size_t)u * D] = h;
        }
        i += (size_t)kHawkUnroll * D;
    }
    for (; t < t1; ++t, i += D) {
        float la, av, v;
        hawk_step(x[i], ga[i], gx[i], csp, la, av, v);
        h = av * h + v;
        y[i] = h;
    }
    if (h_final && ch == nc - 1) h_final[b * D + d] = h;
}

template <typename In>
static hipError_t launch_t(const HawkArgs& a, hipStream_t s) {
    const long n = (long)a.B * a.nc * a.D;
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL((hawk_summary_kernel<In>), dim3(blocks), dim3(256), 0, s, (const In*)a.x, (const In*)a.ga,
                       (const In*)a.gx, a.lam, a.c, a.T, a.D, 0, a.D, a.nc, n, a.Plog, a.S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((hawk_scan_kernel<In>), dim3(blocks), dim3(256), 0, s, (const In*)a.x, (const In*)a.ga,
                       (const In*)a.gx, a.lam, a.c, a.h0, a.T, a.D, 0, a.D, a.nc, n, a.Plog, a.S, a.y, a.h_final);
    return hipGetLastError();
}

hipError_t launch_hawk(const HawkArgs& a, hipStream_t s) {
    return a.bf16 ? launch_t<bf16_t>(a, s) : launch_t<float>(a, s);
}

}  // namespace mesa
