// bwd_adjoint.hip -- the backward's adjoint solve and per-token scalars (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section "A Camada
// Mesa": o_t = G_t (H_t + Lambda)^{-1} q_t with the solve done by CG; the
// bullet "Paralelizacao" says the layer trains in parallel over chunks but
// gives no gradient.  Reading: differentiate o_t implicitly at the forward's
// CG solution x_t, with the adjoint system solved by the same k-step CG on
// the same matrix.  For a loss with dL/do_t = g_t this kernel computes, per
// token of one chunk:
//   bx_t = G_t^T g_t = e^{l_t} (S^G_c)^T g_t + sum_{i=t0..t} e^{l_t - l_i} (v_i . g_t) k_i
//   z_t  = CG(H_t + Lambda, bx_t)                   -> dL/dq_t
//   beta_t = g_t . o_t - z_t . (H_t x_t)            (the query-side gate total)
//   sum over the chunk's tokens of z_t (.) x_t      (minus dL/dlambda, per chunk)
// Work split and layout as the forward CG kernel: one workgroup per (head,
// chunk), wave w owns tokens 16w..16w+15, every product transposed so the
// wave's vectors are the MFMA B operand.  Phase 1 holds (S^G_c)^T, V_c rows
// and K_c^T in LDS for bx; phase 2 holds the stored S^H_c, the mid-chunk
// state, K_c rows and K_c^T for the CG and H_t x_t.
#include "cg_core.h"
#include "mesa_kernels.h"

namespace mesa {

template <int D, int C, int W, typename In>
__device__ __forceinline__ void adjoint_rhs(CgLds<D, C>& L, const CgWave<D, C, W>& cw,
                                            const float* __restrict__ gout, const float* __restrict__ o,
                                            size_t tok0, bool tok_ok, f32x4 (&B)[D / 16], float& go) {
    constexpr int NT = D / 16;
    constexpr int NBO = CgWave<D, C, W>::NBO;
    f32x4 Gv[NT], Ov[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const size_t off = (tok0 + cw.tr) * D + 16 * j + 4 * cw.kk;
        Gv[j] = tok_ok ? *reinterpret_cast<const f32x4*>(gout + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        Ov[j] = tok_ok ? *reinterpret_cast<const f32x4*>(o + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    go = token_dot<NT>(Gv, Ov);
    f32x4 BS[NT], BI[NT], Sc[NBO];
#pragma unroll
    for (int j = 0; j < NT; ++j) BS[j] = BI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < NBO; ++ib) Sc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (S^G_c)^T g (rows of the transposed state) and the scores v_i . g_t
    contract_rows<D, NBO, true>(Gv, L.R, L.KV, cw.n, cw.kk, BS, Sc);
    f32x4 Wg[NBO];
#pragma unroll
    for (int ib = 0; ib < NBO; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Wg[ib][r] = Sc[ib][r] * cw.dec[ib][r];
    contract_intra<D, C, NBO, 0>(Wg, L.KT, cw.n, cw.kk, BI);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) B[j][r] = cw.eLo * BS[j][r] + BI[j][r];
}

template <int D, int C, int W>
__device__ __forceinline__ void adjoint_solve(CgLds<D, C>& L, const CgWave<D, C, W>& cw, f32x4 (&B)[D / 16],
                                              float go, const float* __restrict__ x, size_t tok0, bool tok_ok,
                                              int max_iters, float tol, float* __restrict__ dq,
                                              float* __restrict__ beta, int32_t* __restrict__ z_iters,
                                              f32x4 (&ZX)[D / 16]) {
    constexpr int NT = D / 16;
    f32x4 Z[NT];
    const int it = cg_solve_wave<D, C, W>(L, cw, B, Z, max_iters, tol);
    f32x4 Xv[NT], Hx[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const size_t off = (tok0 + cw.tr) * D + 16 * j + 4 * cw.kk;
        Xv[j] = tok_ok ? *reinterpret_cast<const f32x4*>(x + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    wave_matvec<D, C, W, false>(L, cw, Xv, Hx);
    const float b = go - token_dot<NT>(Z, Hx);
    if (tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
            *reinterpret_cast<f32x4*>(dq + (tok0 + cw.tr) * D + 16 * j + 4 * cw.kk) = Z[j];
        if (cw.kk == 0) {
            beta[tok0 + cw.tr] = b;
            if (z_iters) z_iters[tok0 + cw.tr] = it;
        }
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) ZX[j][r] = Z[j][r] * Xv[j][r];
}

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void bwd_adjoint_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma,
    const float* __restrict__ lambda, const float* __restrict__ x, const float* __restrict__ o,
    const float* __restrict__ gout, const float* __restrict__ SH, const float* __restrict__ SG, int H, int T,
    int n_chunks, int max_iters, float tol, float* __restrict__ dq, float* __restrict__ beta,
    int32_t* __restrict__ z_iters, float* __restrict__ lam_part) {
    constexpr int NW = C / 16;
    constexpr int NT = D / 16;
    constexpr int PS = lds_pitch_rows(D);
    constexpr int NTHR = 64 * NW;
    __shared__ CgLds<D, C> L;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x % n_chunks;
    const long bh = blockIdx.x / n_chunks;
    const int h = (int)(bh % H);
    const int t0 = c * C;
    const int valid = min(C, T - t0);
    const size_t tok0 = (size_t)bh * T + t0;
    constexpr int HPACK = D * (D + 16) / 2;
    const size_t hoff = ((size_t)bh * n_chunks + c) * HPACK;
    const size_t soff = ((size_t)bh * n_chunks + c) * D * D;

    // ---- phase 1: (S^G_c)^T as rows, V_c rows, K_c^T, lambda, l ----
    stage_g_state_transposed<D>(L.R, PS, SG + soff, tid, NTHR);
    stage_chunk_rows<D, C, true, false>(L.KV, nullptr, v + tok0 * D, valid, tid, NTHR);
    stage_chunk_rows<D, C, false, true>(nullptr, L.KT, k + tok0 * D, valid, tid, NTHR);
    for (int e = tid; e < D; e += NTHR) L.Lam[e] = lambda[(size_t)h * D + e];
    if (w == 0) {
        const float l = chunk_log_decay(gamma + tok0, valid, lane);
        if (lane < C) L.L[lane] = l;
    }
    __syncthreads();

    f32x4 B[NT];
    float go = 0.f;
    auto rhs = [&](auto wt) {
        constexpr int WW = decltype(wt)::value;
        const CgWave<D, C, WW> cw(L, lane);
        adjoint_rhs<D, C, WW, In>(L, cw, gout, o, tok0, cw.tr < valid, B, go);
    };
    if (w == 0) rhs(std::integral_constant<int, 0>{});
    else if constexpr (NW > 1) {
        if (w == 1) rhs(std::integral_constant<int, 1>{});
        else if constexpr (NW > 2) {
            if (w == 2) rhs(std::integral_constant<int, 2>{});
            else rhs(std::integral_constant<int, 3>{});
        }
    }
    __syncthreads();   // every wave is done with (S^G_c)^T and V_c

    // ---- phase 2: S^H_c (+ the mid-chunk state), K_c rows ----
    stage_packed_state<D, C>(L, SH + hoff, tid, NTHR);
    stage_chunk_rows<D, C, true, false>(L.KV, nullptr, k + tok0 * D, valid, tid, NTHR);
    __syncthreads();
    if constexpr (NW >= 2) {
        form_mid_state<D, C>(L, w, lane & 15, lane >> 4);
        __syncthreads();
    }

    f32x4 ZX[NT];
    auto solve = [&](auto wt) {
        constexpr int WW = decltype(wt)::value;
        const CgWave<D, C, WW> cw(L, lane);
        adjoint_solve<D, C, WW>(L, cw, B, go, x, tok0, cw.tr < valid, max_iters, tol, dq, beta, z_iters, ZX);
    };
    if (w == 0) solve(std::integral_constant<int, 0>{});
    else if constexpr (NW > 1) {
        if (w == 1) solve(std::integral_constant<int, 1>{});
        else if constexpr (NW > 2) {
            if (w == 2) solve(std::integral_constant<int, 2>{});
            else solve(std::integral_constant<int, 3>{});
        }
    }

    // ---- sum of z (.) x over the chunk's tokens: rows of 16 lanes, then the waves ----
    __syncthreads();   // the K_c rows are no longer read: reuse them as scratch
    float* part = L.KV;   // [NW][D]
    const int kk = lane >> 4;
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float s = rowsum16(ZX[j][r]);
            if ((lane & 15) == 0) part[w * D + 16 * j + 4 * kk + r] = s;
        }
    __syncthreads();
    for (int f = tid; f < D; f += NTHR) {
        float s = 0.f;
        for (int ww = 0; ww < NW; ++ww) s += part[ww * D + f];
        lam_part[((size_t)bh * n_chunks + c) * D + f] = s;
    }
}

template <int D, int C, typename In>
static hipError_t launch_t(const BwdAdjointArgs& a, hipStream_t s) {
    const long grid = a.BH * a.n_chunks;
    hipLaunchKernelGGL((bwd_adjoint_kernel<D, C, In>), dim3((unsigned)grid), dim3(64 * (C / 16)), 0, s,
                       (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.x, a.o, a.gout, a.SH, a.SG, a.H, a.T,
                       a.n_chunks, a.max_iters, a.tol, a.dq, a.beta, a.z_iters, a.lam_part);
    return hipGetLastError();
}

template <int D, typename In>
static hipError_t dispatch_c(const BwdAdjointArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_t<D, 16, In>(a, s);
        case 32: return launch_t<D, 32, In>(a, s);
        case 64: return launch_t<D, 64, In>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename In>
static hipError_t dispatch_d(const BwdAdjointArgs& a, hipStream_t s) {
    switch (a.d) {
        case 16: return dispatch_c<16, In>(a, s);
        case 32: return dispatch_c<32, In>(a, s);
        case 64: return dispatch_c<64, In>(a, s);
        case 128: return dispatch_c<128, In>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_adjoint(const BwdAdjointArgs& a, hipStream_t s) {
    return a.bf16 ? dispatch_d<bf16_t>(a, s) : dispatch_d<float>(a, s);
}

}  // namespace mesa
