// decode.hip -- one recurrent decode step of the Mesa layer (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section "A Camada
// Mesa", bullet "Paralelizacao": inference costs O(1) per token on the state
// variables H_t, G_t; bullet "Computacao Dinamica": the number of CG
// iterations needed to meet the stopping criterion varies per token.  One
// step, per head:
//   H <- gamma H + k k^T,  G <- gamma G + v k^T   (in place)
//   x  = CG on (H + diag lambda) x = q from x0 = 0
//   out = G x
//
// Work split: one 256-thread workgroup per head.  Thread (row, part) keeps
// D/TPR consecutive entries of one row of H in registers for the whole solve,
// so H is read once and written once; the matvec reads p from LDS.  The
// matching entries of G are loaded after the CG: holding only H during the
// solve keeps the kernel at 168 registers, three workgroups per CU, whose
// loads, solves and stores overlap.  The CG scalars are block reductions
// with a fixed order (deterministic), and the stop test is block-uniform.
// The step is bound by HBM traffic on the two d x d states (read + write of
// H and G).
//
// Warm start (section "Significancia e Alegacoes" names warm-start
// strategies as future work): with WARM, each head also carries its previous
// solution x_prev.  The solve starts from x0 = c x_prev with c = 1, or with
// c = x_prev.q / x_prev.(H + Lambda) x_prev (the multiple of x_prev closest to
// the solution in the energy norm; 0 when the denominator is not positive),
// so r0 = q - c (H + Lambda) x_prev; the stop test still compares |r| with
// |q|, a zero q still gives x = 0, and the solution is written back.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

template <int D, bool WARM, typename In>
__global__ __launch_bounds__(256, 3) void decode_kernel(   // three waves per SIMD
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ gamma, const float* __restrict__ lambda, float* __restrict__ SH,
    float* __restrict__ SG, float* __restrict__ SX, int warm_mode, int H, int max_iters, float tol,
    float* __restrict__ out, int32_t* __restrict__ iters) {
    constexpr int TPR = 256 / D;   // threads per state row
    constexpr int EPT = D / TPR;   // state entries per thread
    __shared__ float sq[D], sk[D], sv[D], sp[D], sx[D];
    __shared__ float red[2][4];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wv = tid >> 6;
    const long nh = blockIdx.x;
    const int h = (int)(nh % H);
    const int row = tid / TPR;
    const int part = tid % TPR;
    // Column of this thread's e-th entry: the TPR threads of a row interleave
    // their 4-float pieces, so one 16-byte load instruction of a wave covers
    // TPR * 16 contiguous bytes of each row it touches.
    auto col = [&](int e) {
        if constexpr (EPT % 4 == 0) return (((e >> 2) * TPR + part) << 2) + (e & 3);
        else return part * EPT + e;
    };

    if (tid < D) {
        sq[tid] = to_f32(q[nh * D + tid]);
        sk[tid] = to_f32(k[nh * D + tid]);
        sv[tid] = to_f32(v[nh * D + tid]);
        if constexpr (WARM) sx[tid] = warm_mode != 0 ? SX[nh * D + tid] : 0.f;
    }
    const float g = gamma[nh];
    const float lam_r = lambda[(size_t)h * D + row];
    __syncthreads();

    // Block-wide sum with a fixed reduction order; slot alternates so that a
    // fast thread's next write cannot race a slow thread's read.
    auto block_sum = [&](float val, int slot) {
        val = wavesum(val);
        if (lane == 0) red[slot][wv] = val;
        __syncthreads();
        return (red[slot][0] + red[slot][1]) + (red[slot][2] + red[slot][3]);
    };
    auto row_sum = [&](float val) {
#pragma unroll
        for (int o = 1; o < TPR; o <<= 1) val += __shfl_xor(val, o, 64);
        return val;
    };

    // ---- load this thread's pieces of H; H <- gamma H + k k^T ----
    float hr[EPT];
    float* Hrow = SH + (size_t)nh * D * D + (size_t)row * D;
    float* Grow = SG + (size_t)nh * D * D + (size_t)row * D;
    if constexpr (EPT % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPT; e += 4) {
            const f32x4 x = *reinterpret_cast<const f32x4*>(Hrow + col(e));
#pragma unroll
            for (int u = 0; u < 4; ++u) hr[e + u] = x[u];
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) hr[e] = Hrow[col(e)];
    }
    const float kr = sk[row];
#pragma unroll
    for (int e = 0; e < EPT; ++e) hr[e] = g * hr[e] + kr * sk[col(e)];
    if constexpr (EPT % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPT; e += 4)
            *reinterpret_cast<f32x4*>(Hrow + col(e)) = f32x4{hr[e], hr[e + 1], hr[e + 2], hr[e + 3]};
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) Hrow[col(e)] = hr[e];
    }

    // ---- CG on (H + diag lambda) x = q from x = 0 (or the warm start) ----
    const float q_r = sq[row];
    float x_r = 0.f, r_r = q_r;
    float rr = block_sum(part == 0 ? r_r * r_r : 0.f, 0);
    const float nq = sqrtf(rr);
    if constexpr (WARM) {
        if (warm_mode != 0 && nq > 0.f) {   // block-uniform
            const float xp = sx[row];
            float y = 0.f;
#pragma unroll
            for (int e = 0; e < EPT; ++e) y += hr[e] * sx[col(e)];
            y = row_sum(y) + lam_r * xp;    // (H + Lambda) x_prev
            float c = 1.f;
            if (warm_mode == 2) {
                const float xq = block_sum(part == 0 ? xp * q_r : 0.f, 1);
                const float xax = block_sum(part == 0 ? xp * y : 0.f, 0);
                c = xax > 0.f ? xq / xax : 0.f;
            }
            x_r = c * xp;
            r_r = q_r - c * y;
            rr = block_sum(part == 0 ? r_r * r_r : 0.f, 1);
        }
    }
    float p_r = r_r;
    if (part == 0) sp[row] = p_r;
    __syncthreads();
    int it = 0;
    while (it < max_iters) {
        if ((tol > 0.f && sqrtf(rr) / nq < tol) || rr == 0.f) break;
        float y = 0.f;
#pragma unroll
        for (int e = 0; e < EPT; ++e) y += hr[e] * sp[col(e)];
        y = row_sum(y) + lam_r * p_r;
        const float pap = block_sum(part == 0 ? p_r * y : 0.f, 1);
        if (!(pap > 0.f)) break;
        const float alpha = rr / pap;
        x_r += alpha * p_r;
        r_r -= alpha * y;
        const float rrn = block_sum(part == 0 ? r_r * r_r : 0.f, 0);
        const float beta = rrn / rr;
        p_r = r_r + beta * p_r;
        rr = rrn;
        ++it;
        if (part == 0) sp[row] = p_r;
        __syncthreads();
    }
    // (the warm start's reads of sx ended before the block sums that followed them)
    if (part == 0) {
        sx[row] = x_r;
        if constexpr (WARM) SX[nh * D + row] = x_r;
    }
    __syncthreads();

    // ---- G <- gamma G + v k^T (in place), out = G x ----
    float gr[EPT];
    if constexpr (EPT % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPT; e += 4) {
            const f32x4 y = *reinterpret_cast<const f32x4*>(Grow + col(e));
#pragma unroll
            for (int u = 0; u < 4; ++u) gr[e + u] = y[u];
        }
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) gr[e] = Grow[col(e)];
    }
    const float vr = sv[row];
    float o = 0.f;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        gr[e] = g * gr[e] + vr * sk[col(e)];
        o += gr[e] * sx[col(e)];
    }
    if constexpr (EPT % 4 == 0) {
#pragma unroll
        for (int e = 0; e < EPT; e += 4)
            *reinterpret_cast<f32x4*>(Grow + col(e)) = f32x4{gr[e], gr[e + 1], gr[e + 2], gr[e + 3]};
    } else {
#pragma unroll
        for (int e = 0; e < EPT; ++e) Grow[col(e)] = gr[e];
    }
    o = row_sum(o);
    if (part == 0) out[nh * D + row] = o;
    if (tid == 0 && iters) iters[nh] = it;
}

template <int D, typename In>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t s) {
    if (a.X)
        hipLaunchKernelGGL((decode_kernel<D, true, In>), dim3((unsigned)a.NH), dim3(256), 0, s, (const In*)a.q,
                           (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.SH, a.SG, a.X, a.warm_mode,
                           a.H, a.max_iters, a.tol, a.out, a.iters);
    else
        hipLaunchKernelGGL((decode_kernel<D, false, In>), dim3((unsigned)a.NH), dim3(256), 0, s, (const In*)a.q,
                           (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.SH, a.SG, nullptr, 0, a.H,
                           a.max_iters, a.tol, a.out, a.iters);
    return hipGetLastError();
}

template <typename In>
static hipError_t dispatch_d(const DecodeArgs& a, hipStream_t s) {
    switch (a.d) {
        case 16: return launch_t<16, In>(a, s);
        case 32: return launch_t<32, In>(a, s);
        case 64: return launch_t<64, In>(a, s);
        case 128: return launch_t<128, In>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    return a.bf16 ? dispatch_d<bf16_t>(a, s) : dispatch_d<float>(a, s);
}

}  // namespace mesa
