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
//   sum over the wave's tokens of z_t (.) x_t       (minus dL/dlambda, per chunk and wave)
// Work split and layout as the forward CG kernel (persistent workgroups
// that claim chunks; wave w owns tokens 16w..16w+15; every product
// transposed so the wave's vectors are the MFMA B operand).  For d >= 32
// (both key dtypes) the CG and H_t x_t run on the forward's two-part fp16
// split machinery (cg_h2.h: LDS holds the state and key planes; every
// matvec product on fp16 MFMAs); for d = 16 on fp32 MFMAs with a mid-chunk
// state (cg_core.h).  The right side takes (S^G_c)^T's blocks straight from
// memory (the chunk-state kernel stores them in MFMA operand order for this
// kernel) and the value rows of the scores v_i . g_t from memory too, both
// on fp32 MFMAs, so it needs no LDS of its own; its within-chunk sum goes
// through the staged K^T.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "cg_core.h"
#include "cg_h2.h"
#include "mesa_kernels.h"
#include "persistent.h"

namespace mesa {

// The right side's terms streamed from memory for the wave's tokens, on fp32
// MFMAs: BS = (S^G_c)^T g (B layout), the scores Sc[ib] = v_i . g_t of key
// block ib < W + 1 (accumulator layout: key 16 ib + 4 kk + r, token n), and
// g_t . o_t.
template <int D, int W, typename In>
__device__ __forceinline__ void adjoint_rhs_terms(int n, int kk, int tr, int lane, const ChunkPos& p,
                                                  const In* __restrict__ v, const float* __restrict__ SG,
                                                  const float* __restrict__ gout, const float* __restrict__ o,
                                                  f32x4 (&BS)[D / 16], f32x4 (&Sc)[W + 1], float& go) {
    constexpr int NT = D / 16;
    constexpr int NBO = W + 1;
    const bool tok_ok = tr < p.valid;
    f32x4 Gv[NT];
    {
        f32x4 Ov[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const size_t off = (p.tok0 + tr) * D + 16 * j + 4 * kk;
            Gv[j] = tok_ok ? *reinterpret_cast<const f32x4*>(gout + off) : f32x4{0.f, 0.f, 0.f, 0.f};
            Ov[j] = tok_ok ? *reinterpret_cast<const f32x4*>(o + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        go = token_dot<NT>(Gv, Ov);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) BS[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < NBO; ++ib) Sc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
    // (S^G_c)^T g: this lane's 16 bytes of block (j, g) of (S^G_c)^T are
    // (S^G_c)^T[16j + n][16g + 4kk .. 16g + 4kk + 3].  Scores v_i . g_t: key
    // row 16ib + n, features 16g + 4kk .. + 3, from memory (zero past the end).
    const float* gl = SG + p.soff + 4 * lane;
    constexpr int NB_G = 3;   // block columns in flight: NB_G - 1 steps ahead
    f32x4 ga[NB_G][NT];
    Raw4<In> vb[NB_G][NBO];
    auto gload = [&](int g, int buf) {
#pragma unroll
        for (int j = 0; j < NT; ++j) ga[buf][j] = *reinterpret_cast<const f32x4*>(gl + (j * NT + g) * 256);
#pragma unroll
        for (int ib = 0; ib < NBO; ++ib) {
            const int key = 16 * ib + n;
            vb[buf][ib].zero();
            if (key < p.valid) vb[buf][ib].load(v + (p.tok0 + key) * D + 16 * g + 4 * kk);
        }
    };
#pragma unroll
    for (int g = 0; g < NB_G - 1 && g < NT; ++g) gload(g, g);
#pragma unroll
    for (int g = 0; g < NT; ++g) {
        if (g + NB_G - 1 < NT) gload(g + NB_G - 1, (g + NB_G - 1) % NB_G);
        f32x4 va[NBO];
#pragma unroll
        for (int ib = 0; ib < NBO; ++ib) va[ib] = vb[g % NB_G][ib].get();
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int j = 0; j < NT; ++j) BS[j] = mfma4(ga[g % NB_G][j][s], Gv[g][s], BS[j]);
#pragma unroll
            for (int ib = 0; ib < NBO; ++ib) Sc[ib] = mfma4(va[ib][s], Gv[g][s], Sc[ib]);
        }
    }
}

// B = G_t^T g_t over the wave's tokens (B layout), and g_t . o_t; the
// within-chunk sum through the fp32 K^T tile (d = 16).
template <int D, int C, int W, typename In>
__device__ __forceinline__ void adjoint_rhs(const CgLds<D, C>& L, const CgWave<D, C, W>& cw, int lane,
                                            const ChunkPos& p, const In* __restrict__ v,
                                            const float* __restrict__ SG, const float* __restrict__ gout,
                                            const float* __restrict__ o, f32x4 (&B)[D / 16], float& go) {
    constexpr int NT = D / 16;
    constexpr int NBO = W + 1;
    f32x4 BS[NT], BI[NT], Sc[NBO];
    adjoint_rhs_terms<D, W, In>(cw.n, cw.kk, cw.tr, lane, p, v, SG, gout, o, BS, Sc, go);
    f32x4 Wg[NBO];
#pragma unroll
    for (int ib = 0; ib < NBO; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Wg[ib][r] = Sc[ib][r] * cw.dec[ib][r];
#pragma unroll
    for (int j = 0; j < NT; ++j) BI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    contract_intra<D, C, NBO, 0>(Wg, L.KT, cw.n, cw.kk, BI);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) B[j][r] = cw.eLo * BS[j][r] + BI[j][r];
}

// The same for d >= 32: the decayed scores, split with a per-token exponent,
// go through the staged K^T planes (2^EK) on fp16 MFMAs.
template <int D, int C, int NKP, int W, typename In>
__device__ __forceinline__ void adjoint_rhs_h2(const H2Lds<D, C, NKP>& L, const H2Wave<D, C, W>& wv, int lane,
                                               const ChunkPos& p, const In* __restrict__ v,
                                               const float* __restrict__ SG, const float* __restrict__ gout,
                                               const float* __restrict__ o, int EK, f32x4 (&B)[D / 16], float& go) {
    constexpr int NT = D / 16;
    constexpr int NBO = W + 1;
    constexpr int NS = H2Wave<D, C, W>::NS;
    f32x4 BS[NT], BI[NT], Sc[NBO];
    adjoint_rhs_terms<D, W, In>(wv.n, wv.kk, wv.tr, lane, p, v, SG, gout, o, BS, Sc, go);
    f32x4 Wg[2 * NS];
#pragma unroll
    for (int ib = 0; ib < 2 * NS; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Wg[ib][r] = ib < NBO ? Sc[ib < NBO ? ib : 0][r] * wv.dec[ib][r] : 0.f;
    const int EW = h2_exp(kslot_max(absmax<2 * NS>(Wg)));
#pragma unroll
    for (int j = 0; j < NT; ++j) BI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    h2_apply_kt<D, C, NKP, NS>(L, Wg, pow2(EW), wv.n, wv.kk, BI);
    const float bs = pow2(-(EK + EW));
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) B[j][r] = wv.eLo * BS[j][r] + bs * BI[j][r];
}

// One chunk's work of wave W: right side, adjoint CG, H_t x_t, the per-token
// outputs, and its share of loading and staging the next chunk.  Three
// workgroup barriers: (A) every wave is done with the chunk's LDS tiles;
// (B) the next chunk's S^H, K and gates are staged; (C) its mid-chunk state
// is formed.
template <int D, int C, int W, typename In>
__device__ __forceinline__ bool adjoint_wave(CgLds<D, C>& L, int tid, ChunkPos& p, int n_chunks, int H, int T,
                                             long total, int* __restrict__ work_counter, const In* __restrict__ k,
                                             const In* __restrict__ v, const float* __restrict__ gamma,
                                             const float* __restrict__ lambda, const float* __restrict__ x,
                                             const float* __restrict__ o, const float* __restrict__ gout,
                                             const float* __restrict__ SH, const float* __restrict__ SG,
                                             int max_iters, float tol, float* __restrict__ dq,
                                             float* __restrict__ beta, int32_t* __restrict__ z_iters,
                                             float* __restrict__ lam_part) {
    using CW = CgWave<D, C, W>;
    constexpr int NT = D / 16;
    constexpr int NW = C / 16;
    constexpr int NTHR = 64 * NW;
    constexpr int NLAM = (D + NTHR - 1) / NTHR;
    const int lane = tid & 63;
    const CW cw(L, lane);
    const int kk = cw.kk, tr = cw.tr;
    const bool tok_ok = tr < p.valid;

    // ---- claim this workgroup's next chunk (its number arrives during the CG) ----
    int ticket = 0;
    if (W == 0 && lane == 0) ticket = atomicAdd(work_counter, 1);

    // ---- right side and adjoint CG ----
    f32x4 Bv[NT], Z[NT];
    float go = 0.f;
    adjoint_rhs<D, C, W, In>(L, cw, lane, p, v, SG, gout, o, Bv, go);
    const int it = cg_solve_wave<D, C, W>(L, cw, Bv, Z, max_iters, tol);

    // ---- H_t x_t, beta, dq ----
    f32x4 Xv[NT], Hx[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const size_t off = (p.tok0 + tr) * D + 16 * j + 4 * kk;
        Xv[j] = tok_ok ? *reinterpret_cast<const f32x4*>(x + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    wave_matvec<D, C, W, false>(L, cw, Xv, Hx);
    // Addresses of what follows are built from here on, not held across the CG.
    asm volatile("" : "+v"(tid));
    const float b = go - token_dot<NT>(Z, Hx);
    if (tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
            store_row(dq + (p.tok0 + tr) * D + 16 * j + 4 * kk, Z[j]);
        if (kk == 0) {
            beta[p.tok0 + tr] = b;
            if (z_iters) z_iters[p.tok0 + tr] = it;
        }
    }
    if (W == 0 && lane == 0) L.next = ticket;
    __syncthreads();   // (A) every wave is done with the states, K_c, K_c^T, l and lambda

    // ---- request the next chunk ----
    // Chunks 0..G-1 are the workgroups' first; the claims hand out the rest in order.
    const long nidx = (long)gridDim.x + __builtin_amdgcn_readfirstlane(L.next);
    const bool more = nidx < total;
    const ChunkPos pn = chunk_pos<D, C>(more ? nidx : 0, n_chunks, H, T);
    PackedStateRegs<D, NTHR> nsh;
    ChunkRowsRegs<D, C, NTHR, In> nk;
    float ngam = 1.0f, nlam[NLAM];
    if (more) {
        nsh.load(SH + pn.hoff, tid);
        nk.load(k + pn.tok0 * D, pn.valid, tid);
        if (W == 0) ngam = lane < pn.valid ? gamma[pn.tok0 + lane] : 1.0f;
#pragma unroll
        for (int u = 0; u < NLAM; ++u) {
            const int e = tid + u * NTHR;
            nlam[u] = e < D ? lambda[(size_t)pn.h * D + e] : 0.f;
        }
    }

    // ---- sum over the wave's tokens of z (.) x (lanes n = 0 of each k-slot group) ----
    {
        const size_t chunk = p.soff / ((size_t)D * D);
        float* dst = lam_part + (chunk * NW + W) * D + 4 * kk;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 s;
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] = rowsum16(Z[j][r] * Xv[j][r]);
            if ((lane & 15) == 0) *reinterpret_cast<f32x4*>(dst + 16 * j) = s;
        }
    }
    if (!more) return false;

    // ---- stage the next chunk ----
    nsh.store(L.R, tid);
    nk.store_rows(L.KV, tid);
    nk.store_transposed(L.KT, tid);
    if (W == 0) {
        const float l = chunk_log_decay_of(ngam, pn.valid, lane);
        if (lane < C) L.L[lane] = l;
    }
#pragma unroll
    for (int u = 0; u < NLAM; ++u) {
        const int e = tid + u * NTHR;
        if (e < D) L.Lam[e] = nlam[u];
    }
    __syncthreads();   // (B)
    if constexpr (NW >= 2) {
        form_mid_state<D, C>(L, W, cw.n, kk);
        __syncthreads();   // (C)
    }
    p = pn;
    return true;
}

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void bwd_adjoint_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma,
    const float* __restrict__ lambda, const float* __restrict__ x, const float* __restrict__ o,
    const float* __restrict__ gout, const float* __restrict__ SH, const float* __restrict__ SG, int H, int T,
    int n_chunks, long total, int* __restrict__ work_counter, int max_iters, float tol, float* __restrict__ dq,
    float* __restrict__ beta, int32_t* __restrict__ z_iters, float* __restrict__ lam_part) {
    constexpr int NW = C / 16;
    constexpr int NTHR = 64 * NW;
    __shared__ CgLds<D, C> L;

    const int tid0 = threadIdx.x;
    const int lane = tid0 & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    ChunkPos p = chunk_pos<D, C>(blockIdx.x, n_chunks, H, T);

    // ---- the first chunk: stage S^H_c, K_c (rows and transposed), lambda, l ----
    stage_packed_state<D, C>(L, SH + p.hoff, tid0, NTHR);
    {
        ChunkRowsRegs<D, C, NTHR, In> k0;
        k0.load(k + p.tok0 * D, p.valid, tid0);
        k0.store_rows(L.KV, tid0);
        k0.store_transposed(L.KT, tid0);
    }
    for (int e = tid0; e < D; e += NTHR) L.Lam[e] = lambda[(size_t)p.h * D + e];
    if (w == 0) {
        const float l = chunk_log_decay(gamma + p.tok0, p.valid, lane);
        if (lane < C) L.L[lane] = l;
    }
    __syncthreads();
    if constexpr (NW >= 2) {
        form_mid_state<D, C>(L, w, lane & 15, lane >> 4);
        __syncthreads();
    }

    for (bool more = true; more;) {
        // An opaque copy of the thread id: the per-lane LDS addresses derived
        // from it are rebuilt per chunk instead of being held in registers.
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        auto body = [&](auto wt) {
            constexpr int WW = decltype(wt)::value;
            return adjoint_wave<D, C, WW, In>(L, tid, p, n_chunks, H, T, total, work_counter, k, v, gamma, lambda,
                                              x, o, gout, SH, SG, max_iters, tol, dq, beta, z_iters, lam_part);
        };
        if (w == 0) more = body(std::integral_constant<int, 0>{});
        else if constexpr (NW > 1) {
            if (w == 1) more = body(std::integral_constant<int, 1>{});
            else if constexpr (NW > 2) {
                if (w == 2) more = body(std::integral_constant<int, 2>{});
                else more = body(std::integral_constant<int, 3>{});
            }
        }
    }
}

// ---------------------------------------------------------------------------
// d >= 32: the adjoint CG and H_t x_t on the forward's two-part fp16 split
// machinery (cg_h2.h).  Three workgroup barriers per chunk: (A) every wave
// is done with the LDS planes; (B) the next chunk's maxima, gates and lambda
// are in; (C) its state and key planes are staged.
template <int D, int C, int W, typename In>
__device__ __forceinline__ bool adjoint_h2_wave(H2Lds<D, C, h2_key_planes<In>()>& L, int tid, ChunkPos& p, int& ES,
                                                int& EK, int n_chunks, int H, int T, long total,
                                                int* __restrict__ work_counter, const In* __restrict__ k,
                                                const In* __restrict__ v, const float* __restrict__ gamma,
                                                const float* __restrict__ lambda, const float* __restrict__ x,
                                                const float* __restrict__ o, const float* __restrict__ gout,
                                                const float* __restrict__ SH, const float* __restrict__ SG,
                                                int max_iters, float tol, float* __restrict__ dq,
                                                float* __restrict__ beta, int32_t* __restrict__ z_iters,
                                                float* __restrict__ lam_part) {
    constexpr int NKP = h2_key_planes<In>();
    using Wv = H2Wave<D, C, W>;
    constexpr int NT = D / 16;
    constexpr int NW = C / 16;
    constexpr int NTHR = 64 * NW;
    constexpr int NLAM = (D + NTHR - 1) / NTHR;
    const int lane = tid & 63;
    const Wv wv(L.L, lane);
    const int kk = wv.kk, tr = wv.tr;
    const bool tok_ok = tr < p.valid;

    int ticket = 0;
    if (W == 0 && lane == 0) ticket = atomicAdd(work_counter, 1);

    // ---- right side and adjoint CG ----
    f32x4 Bv[NT], Z[NT], lam[NT];
    float go = 0.f;
    adjoint_rhs_h2<D, C, NKP, W, In>(L, wv, lane, p, v, SG, gout, o, EK, Bv, go);
#pragma unroll
    for (int j = 0; j < NT; ++j) lam[j] = lds4(&L.Lam[16 * j + 4 * kk]);
    H2Hi<D, NKP> SHr;   // unused: the solve reads the hi plane itself
    const int it = h2_cg_solve<D, C, NKP, W, 0, false>(L, wv, ES, EK, Bv, Z, lam, max_iters, tol, L.S[1], SHr);

    // ---- H_t x_t, beta, dq ----
    f32x4 Xv[NT], Hx[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const size_t off = (p.tok0 + tr) * D + 16 * j + 4 * kk;
        Xv[j] = tok_ok ? *reinterpret_cast<const f32x4*>(x + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    h2_matvec<D, C, NKP, W>(L, wv, ES, EK, Xv, Hx);
    asm volatile("" : "+v"(tid));
    const float b = go - token_dot<NT>(Z, Hx);
    if (tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
            store_row(dq + (p.tok0 + tr) * D + 16 * j + 4 * kk, Z[j]);
        if (kk == 0) {
            beta[p.tok0 + tr] = b;
            if (z_iters) z_iters[p.tok0 + tr] = it;
        }
    }
    if (W == 0 && lane == 0) L.next = ticket;
    __syncthreads();   // (A) every wave is done with the state and key planes, l and lambda

    const long nidx = (long)gridDim.x + __builtin_amdgcn_readfirstlane(L.next);
    const bool more = nidx < total;
    const ChunkPos pn = chunk_pos<D, C>(more ? nidx : 0, n_chunks, H, T);
    PackedStateRegs<D, NTHR> nsh;
    ChunkRowsRegs<D, C, NTHR, In> nk;
    float ngam = 1.0f, nlam[NLAM];
    if (more) {
        nsh.load(SH + pn.hoff, tid);
        nk.load(k + pn.tok0 * D, pn.valid, tid);
        if (W == 0) ngam = lane < pn.valid ? gamma[pn.tok0 + lane] : 1.0f;
#pragma unroll
        for (int u = 0; u < NLAM; ++u) {
            const int e = tid + u * NTHR;
            nlam[u] = e < D ? lambda[(size_t)pn.h * D + e] : 0.f;
        }
    }

    // ---- sum over the wave's tokens of z (.) x (lanes n = 0 of each k-slot group) ----
    {
        const size_t chunk = p.soff / ((size_t)D * D);
        float* dst = lam_part + (chunk * NW + W) * D + 4 * kk;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 s;
#pragma unroll
            for (int r = 0; r < 4; ++r) s[r] = rowsum16(Z[j][r] * Xv[j][r]);
            if ((lane & 15) == 0) *reinterpret_cast<f32x4*>(dst + 16 * j) = s;
        }
    }
    if (!more) return false;

    // ---- stage the next chunk ----
    h2_put_maxima<D, C, NTHR, NKP, In>(L, nsh, nk, tid, lane, W);
    if (W == 0) {
        const float l = chunk_log_decay_of(ngam, pn.valid, lane);
        if (lane < C) L.L[lane] = l;
    }
#pragma unroll
    for (int u = 0; u < NLAM; ++u) {
        const int e = tid + u * NTHR;
        if (e < D) L.Lam[e] = nlam[u];
    }
    __syncthreads();   // (B)
    h2_stage_chunk<D, C, NTHR, NKP, In>(L, nsh, nk, tid, ES, EK);
    __syncthreads();   // (C)
    p = pn;
    return true;
}

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void bwd_adjoint_h2_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma,
    const float* __restrict__ lambda, const float* __restrict__ x, const float* __restrict__ o,
    const float* __restrict__ gout, const float* __restrict__ SH, const float* __restrict__ SG, int H, int T,
    int n_chunks, long total, int* __restrict__ work_counter, int max_iters, float tol, float* __restrict__ dq,
    float* __restrict__ beta, int32_t* __restrict__ z_iters, float* __restrict__ lam_part) {
    constexpr int NKP = h2_key_planes<In>();
    constexpr int NW = C / 16;
    constexpr int NTHR = 64 * NW;
    __shared__ H2Lds<D, C, NKP> L;

    const int tid0 = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    ChunkPos p = chunk_pos<D, C>(blockIdx.x, n_chunks, H, T);
    int ES, EK;
    h2_stage_first<D, C, NTHR, NKP, In>(L, p, SH, k, gamma, lambda, tid0, ES, EK);

    for (bool more = true; more;) {
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        auto body = [&](auto wt) {
            constexpr int WW = decltype(wt)::value;
            return adjoint_h2_wave<D, C, WW, In>(L, tid, p, ES, EK, n_chunks, H, T, total, work_counter, k, v, gamma,
                                                 lambda, x, o, gout, SH, SG, max_iters, tol, dq, beta, z_iters,
                                                 lam_part);
        };
        if (w == 0) more = body(std::integral_constant<int, 0>{});
        else if constexpr (NW > 1) {
            if (w == 1) more = body(std::integral_constant<int, 1>{});
            else if constexpr (NW > 2) {
                if (w == 2) more = body(std::integral_constant<int, 2>{});
                else more = body(std::integral_constant<int, 3>{});
            }
        }
    }
}

template <int D, int C, typename In>
static hipError_t launch_fp32_keys(const BwdAdjointArgs& a, hipStream_t s);

template <int D, int C, typename In>
static hipError_t launch_t(const BwdAdjointArgs& a, hipStream_t s) {
    if constexpr (D >= 32) {
        static std::atomic<long> resident_h2[kMaxDevices];
        const long total = a.BH * a.n_chunks;
        const int block = 64 * (C / 16);
        const long grid = std::min(total, resident_workgroups(bwd_adjoint_h2_kernel<D, C, In>, block, resident_h2));
        hipLaunchKernelGGL((bwd_adjoint_h2_kernel<D, C, In>), dim3((unsigned)grid), dim3(block), 0, s,
                           (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.x, a.o, a.gout, a.SH, a.SG, a.H,
                           a.T, a.n_chunks, total, a.work_counter, a.max_iters, a.tol, a.dq, a.beta, a.z_iters,
                           a.lam_part);
        return hipGetLastError();
    } else {
        return launch_fp32_keys<D, C, In>(a, s);
    }
}

template <int D, int C, typename In>
static hipError_t launch_fp32_keys(const BwdAdjointArgs& a, hipStream_t s) {
    static std::atomic<long> resident[kMaxDevices];
    const long total = a.BH * a.n_chunks;
    const int block = 64 * (C / 16);
    const long grid = std::min(total, resident_workgroups(bwd_adjoint_kernel<D, C, In>, block, resident));
    hipLaunchKernelGGL((bwd_adjoint_kernel<D, C, In>), dim3((unsigned)grid), dim3(block), 0, s,
                       (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.x, a.o, a.gout, a.SH, a.SG, a.H, a.T,
                       a.n_chunks, total, a.work_counter, a.max_iters, a.tol, a.dq, a.beta, a.z_iters, a.lam_part);
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
