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
// state and rescans the chunk, writing h.  A thread owns four consecutive
// channels (one 8- or 16-byte piece per row; one channel when rows or
// pointers are not aligned for that) of one chunk; consecutive threads take
// consecutive channels, so every load and store of a wave is one contiguous
// row piece.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

constexpr int kHawkUnroll = 8;

__device__ __forceinline__ float hawk_softplus(float z) { return z > 20.f ? z : log1pf(__expf(z)); }
// The gates and the input scale use the hardware reciprocal and square root
// (about 1 ulp each) instead of correctly rounded division and sqrt
// sequences: those made the scan ALU-bound.
__device__ __forceinline__ float hawk_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// V consecutive channels of one row, loaded as one 4V- or 2V-byte piece
// (V = 1: a single element).
template <typename In, int V> struct HawkVec;
template <typename In> struct HawkVec<In, 1> {
    In v[1];
    __device__ __forceinline__ void load(const In* p) { v[0] = *p; }
    __device__ __forceinline__ float get(int) const { return to_f32(v[0]); }
};
template <> struct HawkVec<float, 4> {
    f32x4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};
template <> struct HawkVec<bf16_t, 4> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t w = i < 2 ? v.x : v.y;
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

template <int V>
__device__ __forceinline__ void store_v(float* p, const float (&x)[V]) {
    if constexpr (V == 4) *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    else p[0] = x[0];
}

// One step's decay (as its log and value) and input term.  1 - a^2 is the
// short Taylor series of 1 - e^{2 log a} where the subtraction would cancel
// (2 log a > -1/16: the first dropped term is below 2^-24 relative), and
// 1 - a*a elsewhere (a < 0.97, so 1 - a*a > 0.06 keeps ~23 bits).
__device__ __forceinline__ void hawk_step_f(float xv, float gav, float gxv, float csp, float& loga, float& a,
                                            float& u) {
    const float r = hawk_sigmoid(gav);
    const float i = hawk_sigmoid(gxv);
    loga = -csp * r;
    a = __expf(loga);
    const float z = 2.0f * loga;
    const float taylor = -z * (1.f + z * (0.5f + z * (1.f / 6.f + z * (1.f / 24.f + z * (1.f / 120.f)))));
    const float oma = z > -0.0625f ? taylor : 1.f - a * a;
    u = __builtin_amdgcn_sqrtf(oma) * (i * xv);
}

// A thread owns channels d .. d+V-1 of one chunk of one sequence.
template <typename In, int V>
__global__ __launch_bounds__(256) void hawk_summary_kernel(const In* __restrict__ x, const In* __restrict__ ga,
                                                           const In* __restrict__ gx, const float* __restrict__ lam,
                                                           float c, int T, int D, int nc, long n_threads,
                                                           float* __restrict__ Plog, float* __restrict__ S) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= n_threads) return;
    const int DV = D / V;
    const int d = V * (int)(g % DV);
    const long rem = g / DV;
    const int ch = (int)(rem % nc);
    const long b = rem / nc;
    const int t0 = ch * kHawkChunk, t1 = min(T, t0 + kHawkChunk);
    float csp[V], h[V], lsum[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        csp[q] = c * hawk_softplus(-lam[d + q]);
        h[q] = 0.f;
        lsum[q] = 0.f;
    }
    size_t i = ((size_t)b * T + t0) * D + d;
    int t = t0;
    for (; t + kHawkUnroll <= t1; t += kHawkUnroll) {
        HawkVec<In, V> xr[kHawkUnroll], ar[kHawkUnroll], gr[kHawkUnroll];
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            xr[u].load(x + i + (size_t)u * D);
            ar[u].load(ga + i + (size_t)u * D);
            gr[u].load(gx + i + (size_t)u * D);
        }
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u)
#pragma unroll
            for (int q = 0; q < V; ++q) {
                float la, av, vv;
                hawk_step_f(xr[u].get(q), ar[u].get(q), gr[u].get(q), csp[q], la, av, vv);
                h[q] = av * h[q] + vv;
                lsum[q] += la;
            }
        i += (size_t)kHawkUnroll * D;
    }
    for (; t < t1; ++t, i += D) {
        HawkVec<In, V> xr, ar, gr;
        xr.load(x + i);
        ar.load(ga + i);
        gr.load(gx + i);
#pragma unroll
        for (int q = 0; q < V; ++q) {
            float la, av, vv;
            hawk_step_f(xr.get(q), ar.get(q), gr.get(q), csp[q], la, av, vv);
            h[q] = av * h[q] + vv;
            lsum[q] += la;
        }
    }
    const size_t j = ((size_t)b * nc + ch) * D + d;
    store_v<V>(Plog + j, lsum);   // log of the chunk's decay product
    store_v<V>(S + j, h);         // the chunk's end state from zero
}

template <typename In, int V>
__global__ __launch_bounds__(256) void hawk_scan_kernel(const In* __restrict__ x, const In* __restrict__ ga,
                                                        const In* __restrict__ gx, const float* __restrict__ lam,
                                                        float c, const float* __restrict__ h0, int T, int D, int nc,
                                                        long n_threads, const float* __restrict__ Plog,
                                                        const float* __restrict__ S, float* __restrict__ y,
                                                        float* __restrict__ h_final) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= n_threads) return;
    const int DV = D / V;
    const int d = V * (int)(g % DV);
    const long rem = g / DV;
    const int ch = (int)(rem % nc);
    const long b = rem / nc;
    const int t0 = ch * kHawkChunk, t1 = min(T, t0 + kHawkChunk);
    float csp[V], h[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        csp[q] = c * hawk_softplus(-lam[d + q]);
        h[q] = h0 ? h0[b * D + d + q] : 0.f;
    }
    // the chunk's start state: fold the earlier chunks' (P, s) in order,
    // eight summaries requested at a time
    {
        const size_t j0 = (size_t)b * nc * D + d;
        int cc = 0;
        for (; cc + 8 <= ch; cc += 8) {
            HawkVec<float, V> pl[8], sv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                pl[u].load(Plog + j0 + (size_t)(cc + u) * D);
                sv[u].load(S + j0 + (size_t)(cc + u) * D);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int q = 0; q < V; ++q) h[q] = __expf(pl[u].get(q)) * h[q] + sv[u].get(q);
        }
        for (; cc < ch; ++cc) {
            HawkVec<float, V> pl, sv;
            pl.load(Plog + j0 + (size_t)cc * D);
            sv.load(S + j0 + (size_t)cc * D);
#pragma unroll
            for (int q = 0; q < V; ++q) h[q] = __expf(pl.get(q)) * h[q] + sv.get(q);
        }
    }
    size_t i = ((size_t)b * T + t0) * D + d;
    int t = t0;
    for (; t + kHawkUnroll <= t1; t += kHawkUnroll) {
        HawkVec<In, V> xr[kHawkUnroll], ar[kHawkUnroll], gr[kHawkUnroll];
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            xr[u].load(x + i + (size_t)u * D);
            ar[u].load(ga + i + (size_t)u * D);
            gr[u].load(gx + i + (size_t)u * D);
        }
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            float out[V];
#pragma unroll
            for (int q = 0; q < V; ++q) {
                float la, av, vv;
                hawk_step_f(xr[u].get(q), ar[u].get(q), gr[u].get(q), csp[q], la, av, vv);
                h[q] = av * h[q] + vv;
                out[q] = h[q];
            }
            store_v<V>(y + i + (size_t)u * D, out);
        }
        i += (size_t)kHawkUnroll * D;
    }
    for (; t < t1; ++t, i += D) {
        HawkVec<In, V> xr, ar, gr;
        xr.load(x + i);
        ar.load(ga + i);
        gr.load(gx + i);
        float out[V];
#pragma unroll
        for (int q = 0; q < V; ++q) {
            float la, av, vv;
            hawk_step_f(xr.get(q), ar.get(q), gr.get(q), csp[q], la, av, vv);
            h[q] = av * h[q] + vv;
            out[q] = h[q];
        }
        store_v<V>(y + i, out);
    }
    if (h_final && ch == nc - 1) store_v<V>(h_final + b * D + d, h);
}

template <typename In, int V>
static hipError_t launch_t(const HawkArgs& a, hipStream_t s) {
    const long n = (long)a.B * a.nc * (a.D / V);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL((hawk_summary_kernel<In, V>), dim3(blocks), dim3(256), 0, s, (const In*)a.x,
                       (const In*)a.ga, (const In*)a.gx, a.lam, a.c, a.T, a.D, a.nc, n, a.Plog, a.S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((hawk_scan_kernel<In, V>), dim3(blocks), dim3(256), 0, s, (const In*)a.x, (const In*)a.ga,
                       (const In*)a.gx, a.lam, a.c, a.h0, a.T, a.D, a.nc, n, a.Plog, a.S, a.y, a.h_final);
    return hipGetLastError();
}

// Four channels per thread (one 8- or 16-byte piece per row) when the rows
// and pointers allow it, else one.
hipError_t launch_hawk(const HawkArgs& a, hipStream_t s) {
    const size_t esz = a.bf16 ? 2 : 4;
    auto al = [&](const void* p, size_t n) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % n == 0; };
    const bool vec = a.D % 4 == 0 && al(a.x, 4 * esz) && al(a.ga, 4 * esz) && al(a.gx, 4 * esz) && al(a.y, 16) &&
                     al(a.h0, 16) && al(a.h_final, 16) && al(a.lam, 16) && al(a.Plog, 16) && al(a.S, 16);
    if (a.bf16) return vec ? launch_t<bf16_t, 4>(a, s) : launch_t<bf16_t, 1>(a, s);
    return vec ? launch_t<float, 4>(a, s) : launch_t<float, 1>(a, s);
}

}  // namespace mesa
