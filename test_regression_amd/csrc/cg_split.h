// cg_split.h -- the forward CG kernel's chunk machinery for bf16 keys
// (gfx950): every product of the CG matvec runs on bf16 MFMAs.
//
// MesaNet summary page (gist.science, paper 2506.05233), section "A Camada
// Mesa", bullet "Paralelizacao": the CG over all time steps is a gated-
// linear-attention pass run chunk-parallel on the states.  For chunk c
// (tokens t0..t0+C-1, l_t the within-chunk prefix sum of ln gamma,
// S = S^H_c = H_{t0-1}):
//   H_t p = e^{l_t} S p + sum_{i=t0..t} e^{l_t - l_i} (k_i . p) k_i
//
// Exact split products.  A float x is split by truncation into three bf16
// parts hi + mid + lo = x (split_operands in cg_core.h).  The chunk state S
// is held in LDS as the three bf16 planes of its split (the full matrix, so
// every A operand is a row read); the keys are exact bf16.  The state term
// S p takes all nine products of S's planes with p's parts and the
// intra-chunk terms three products of the exact keys with the parts of p or
// of the decayed scores, so every product term is the exact float product
// and only the order of the sums differs from an fp32 contraction.
//
// LDS layout.  A 32-slot MFMA operand (v_mfma_f32_16x16x32_bf16) of lane
// group kk is the 4-element pieces 4kk..4kk+3 of two 16-column blocks (the
// CG vectors hold exactly these in registers).  Rows of the state planes and
// of the key tiles store each 32-column block permuted so that those eight
// columns are contiguous (perm32): a lane's operand is one 128-bit read.  Row
// pitches are 8 words more than the row (an odd multiple of 8 words), so the
// 16-byte pieces that rows m = 0..7 and lane groups kk = 0, 1 read fall on
// distinct banks.
#pragma once
#include "cg_core.h"

namespace mesa {

// Position of column c within its 32-column block after the permutation.
__host__ __device__ constexpr int perm32(int c) {
    return 32 * (c / 32) + 8 * ((c % 16) / 4) + 4 * ((c % 32) / 16) + (c % 4);
}

template <int D, int C>
struct alignas(16) SplitLds {
    static constexpr int SW = D / 2 + 8;                    // words per state / key row
    static constexpr int KW = (C >= 32 ? C : 32) / 2 + 8;   // words per K^T row (at least one 32-key step)
    uint32_t S[3][D * SW];   // S^H_c: bf16 planes hi, mid, lo; row r = feature r, columns perm32
    uint32_t KR[C * SW];     // K_c rows (bf16, columns perm32)
    uint32_t KT[D * KW];     // K_c^T, later V_c^T (bf16, tokens perm32)
    float L[C];              // l_i
    float Lam[D];
    int next;                // the claimed next chunk
};

__device__ __forceinline__ bf16x8 lds_bf16x8(const uint32_t* p) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    return as_bf16x8(w);
}

// Per-wave constants of wave W.
template <int D, int C, int W>
struct SplitWave {
    static constexpr int NT = D / 16;
    static constexpr int NW = C / 16;
    static constexpr int NBO = W + 1;          // causal key blocks from the chunk start
    static constexpr int NS = (NBO + 1) / 2;   // 32-key steps of the intra-chunk apply
    int n, kk, tr;
    float eLo;                 // e^{l_t}
    float dec[2 * NS][4];      // e^{l_t - l_i}, key i = 16 ib + 4kk + r <= t, else 0
    __device__ __forceinline__ SplitWave(const SplitLds<D, C>& L, int lane) {
        n = lane & 15;
        kk = lane >> 4;
        tr = 16 * W + n;
        eLo = __expf(L.L[tr]);
#pragma unroll
        for (int ib = 0; ib < 2 * NS; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ib + 4 * kk + r;
                dec[ib][r] = (i <= tr) ? __expf(L.L[tr] - L.L[i < C ? i : C - 1]) : 0.f;
            }
    }
};

// The A operand of K^T (or V^T) row block j for 32-key step s; the second
// 16 keys are zero when the chunk has no such block (C = 16).
template <int D, int C>
__device__ __forceinline__ bf16x8 kt_operand(const SplitLds<D, C>& L, int j, int s, int m, int kk) {
    constexpr int KW = SplitLds<D, C>::KW;
    if constexpr (C >= 32) {
        return lds_bf16x8(&L.KT[(16 * j + m) * KW + 16 * s + 4 * kk]);
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(&L.KT[(16 * j + m) * KW + 4 * kk]);
        const uint32_t w[4] = {v.x, v.y, 0u, 0u};
        return as_bf16x8(w);
    }
}

// Sc[ib] = K[16 ib + m][:] . Z^T[:][n] (ib < NB), exact-bf16 keys times the
// split of Z; Zs holds the split parts of Z per 32-feature step.
template <int D, int C, int NB>
__device__ __forceinline__ void split_scores(const SplitLds<D, C>& L, const bf16x8 (&Zs)[D / 32][3], int m, int kk,
                                             f32x4 (&Sc)[NB]) {
    constexpr int SW = SplitLds<D, C>::SW;
#pragma unroll
    for (int q = 0; q < D / 32; ++q)
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) {
            const bf16x8 A = lds_bf16x8(&L.KR[(16 * ib + m) * SW + 16 * q + 4 * kk]);
            Sc[ib] = mfma_bf16x32(A, Zs[q][2], Sc[ib]);
            Sc[ib] = mfma_bf16x32(A, Zs[q][1], Sc[ib]);
            Sc[ib] = mfma_bf16x32(A, Zs[q][0], Sc[ib]);
        }
}

// Y[j] += sum_i T[16j + m][i] W[i][n] over NS 32-key steps of the K^T / V^T
// tile, W the decayed scores (split here).
template <int D, int C, int NS>
__device__ __forceinline__ void split_apply(const SplitLds<D, C>& L, const f32x4 (&W)[2 * NS], int m, int kk,
                                            f32x4 (&Y)[D / 16]) {
    constexpr int NT = D / 16;
    constexpr int JI = NT >= 4 ? 4 : NT;   // row blocks whose chains interleave
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        bf16x8 Wp[3];
        split_operands(W[2 * s], W[2 * s + 1], Wp[0], Wp[1], Wp[2]);
#pragma unroll
        for (int j = 0; j < NT; j += JI) {
            bf16x8 A[JI];
#pragma unroll
            for (int h = 0; h < JI; ++h) A[h] = kt_operand<D, C>(L, j + h, s, m, kk);
#pragma unroll
            for (int t = 2; t >= 0; --t)
#pragma unroll
                for (int h = 0; h < JI; ++h) Y[j + h] = mfma_bf16x32(A[h], Wp[t], Y[j + h]);
        }
    }
}

// One CG matvec of wave W: YS = S P^T (nine split products per step), and
// YI = K^T (M o (K P^T)) over the causal keys from the chunk start.  head()
// starts it from P's first two 16-feature blocks alone (their split and the
// first scores step), so the CG loop can issue it before it has finished
// updating the rest of P; rest() completes it.  Order inside: per
// 32-feature step q the split of P, the scores and the state products; the
// last two steps' scores come before the second-to-last state step, so that
// the decayed scores are split under its MFMAs; then the apply, then the
// last state step.
template <int D, int C, int W>
struct SplitMatvec {
    using SWv = SplitWave<D, C, W>;
    static constexpr int NT = D / 16;
    static constexpr int NQ = D / 32;
    static constexpr int SW = SplitLds<D, C>::SW;
    // JI row blocks at a time, their nine products interleaved, so that
    // consecutive MFMAs never wait on each other's accumulator; the next
    // group's state rows are read while the current group's products run.
    static constexpr int JI = NT >= 2 ? 2 : NT;
    static constexpr int NG = NT / JI;
    const SplitLds<D, C>& L;
    const SWv& sw;
    // Scores: one accumulator per key block, and per split part too when a
    // single key block would otherwise make one dependent chain.
    static constexpr int NP = SWv::NBO == 1 ? 3 : 1;
    f32x4 Sp[SWv::NBO][NP];
    bf16x8 Z0[3];            // split of P's first 32 features

    __device__ __forceinline__ SplitMatvec(const SplitLds<D, C>& l, const SWv& w) : L(l), sw(w) {}

    __device__ __forceinline__ static void split_step(const f32x4 (&P)[NT], int q, bf16x8 (&Z)[3]) {
        split_operands(P[2 * q], P[2 * q + 1], Z[0], Z[1], Z[2]);
    }
    __device__ __forceinline__ void scores_step(int q, const bf16x8 (&Z)[3]) {
        bf16x8 A[SWv::NBO];
#pragma unroll
        for (int ib = 0; ib < SWv::NBO; ++ib) A[ib] = lds_bf16x8(&L.KR[(16 * ib + sw.n) * SW + 16 * q + 4 * sw.kk]);
#pragma unroll
        for (int t = 2; t >= 0; --t)
#pragma unroll
            for (int ib = 0; ib < SWv::NBO; ++ib)
                Sp[ib][NP == 3 ? t : 0] = mfma_bf16x32(A[ib], Z[t], Sp[ib][NP == 3 ? t : 0]);
    }
    __device__ __forceinline__ void load_group(int q, int g, bf16x8 (&A)[JI][3]) const {
#pragma unroll
        for (int h = 0; h < JI; ++h) {
            const int off = (16 * (g * JI + h) + sw.n) * SW + 16 * q + 4 * sw.kk;
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) A[h][pl] = lds_bf16x8(&L.S[pl][off]);
        }
    }
    __device__ __forceinline__ void state_step(int q, const bf16x8 (&Z)[3], f32x4 (&YS)[NT]) const {
        bf16x8 A[2][JI][3];
        load_group(q, 0, A[0]);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) load_group(q, g + 1, A[(g + 1) & 1]);
            // smallest terms first: (plane, part) = (2,2) (2,1) (1,2) (2,0) (1,1) (0,2) (1,0) (0,1) (0,0)
            constexpr int PL[9] = {2, 2, 1, 2, 1, 0, 1, 0, 0};
            constexpr int PT[9] = {2, 1, 2, 0, 1, 2, 0, 1, 0};
#pragma unroll
            for (int t = 0; t < 9; ++t)
#pragma unroll
                for (int h = 0; h < JI; ++h)
                    YS[g * JI + h] = mfma_bf16x32(A[g & 1][h][PL[t]], Z[PT[t]], YS[g * JI + h]);
        }
    }
    __device__ __forceinline__ void apply(f32x4 (&YI)[NT]) const {
        f32x4 Wt[2 * SWv::NS];
#pragma unroll
        for (int ib = 0; ib < 2 * SWv::NS; ++ib) {
            const int b = ib < SWv::NBO ? ib : 0;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                float sc = Sp[b][0][r];
                if constexpr (NP == 3) sc = (Sp[b][2][r] + Sp[b][1][r]) + Sp[b][0][r];
                Wt[ib][r] = ib < SWv::NBO ? sc * sw.dec[ib][r] : 0.f;
            }
        }
        split_apply<D, C, SWv::NS>(L, Wt, sw.n, sw.kk, YI);
    }

    __device__ __forceinline__ void head(const f32x4 (&P)[NT]) {
        const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ib = 0; ib < SWv::NBO; ++ib)
#pragma unroll
            for (int t = 0; t < NP; ++t) Sp[ib][t] = zero;
        split_step(P, 0, Z0);
        scores_step(0, Z0);
    }

    __device__ __forceinline__ void rest(const f32x4 (&P)[NT], f32x4 (&YS)[NT], f32x4 (&YI)[NT]) {
        const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j) YS[j] = YI[j] = zero;
        if constexpr (NQ == 1) {
            apply(YI);
            state_step(0, Z0, YS);
        } else {
            bf16x8 Za[3], Zb[3];
            if constexpr (NQ == 2) {
                split_step(P, 1, Zb);
                scores_step(1, Zb);
                state_step(0, Z0, YS);
            } else {
                state_step(0, Z0, YS);
#pragma unroll
                for (int q = 1; q + 2 < NQ; ++q) {
                    split_step(P, q, Za);
                    scores_step(q, Za);
                    state_step(q, Za, YS);
                }
                split_step(P, NQ - 2, Za);
                split_step(P, NQ - 1, Zb);
                scores_step(NQ - 2, Za);
                scores_step(NQ - 1, Zb);
                state_step(NQ - 2, Za, YS);
            }
            apply(YI);
            state_step(NQ - 1, Zb, YS);
        }
    }
};

// One whole matvec as a single function (the adjoint kernel; its loop was
// slower with SplitMatvec's head/rest form): YS = S P^T (nine split
// products per step), and
// YI = K^T (M o (K P^T)) over the causal keys from the chunk start.  Order:
// per 32-feature step q the split of P, the scores and the state products;
// the last two steps' scores come before the second-to-last state step, so
// that the decayed scores are split under its MFMAs; then the apply, then
// the last state step, whose MFMAs complete the state blocks one by one so
// that the CG update of block j can start while later blocks still run.
template <int D, int C, int W>
__device__ __forceinline__ void split_matvec(const SplitLds<D, C>& L, const SplitWave<D, C, W>& sw,
                                             const f32x4 (&P)[D / 16], f32x4 (&YS)[D / 16], f32x4 (&YI)[D / 16]) {
    using SWv = SplitWave<D, C, W>;
    constexpr int NT = D / 16;
    constexpr int NQ = D / 32;
    constexpr int SW = SplitLds<D, C>::SW;
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    // scores: one accumulator per key block and split part (independent chains)
    f32x4 Sp[SWv::NBO][3];
#pragma unroll
    for (int ib = 0; ib < SWv::NBO; ++ib) Sp[ib][0] = Sp[ib][1] = Sp[ib][2] = zero;
#pragma unroll
    for (int j = 0; j < NT; ++j) YS[j] = YI[j] = zero;
    auto split_step = [&](int q, bf16x8 (&Z)[3]) { split_operands(P[2 * q], P[2 * q + 1], Z[0], Z[1], Z[2]); };
    auto scores_step = [&](int q, const bf16x8 (&Z)[3]) {
        bf16x8 A[SWv::NBO];
#pragma unroll
        for (int ib = 0; ib < SWv::NBO; ++ib) A[ib] = lds_bf16x8(&L.KR[(16 * ib + sw.n) * SW + 16 * q + 4 * sw.kk]);
#pragma unroll
        for (int t = 2; t >= 0; --t)
#pragma unroll
            for (int ib = 0; ib < SWv::NBO; ++ib) Sp[ib][t] = mfma_bf16x32(A[ib], Z[t], Sp[ib][t]);
    };
    // JI row blocks at a time, their nine products interleaved, so that
    // consecutive MFMAs never wait on each other's accumulator; the next
    // group's state rows are read while the current group's products run.
    constexpr int JI = NT >= 2 ? 2 : NT;
    constexpr int NG = NT / JI;
    auto load_group = [&](int q, int g, bf16x8 (&A)[JI][3]) {
#pragma unroll
        for (int h = 0; h < JI; ++h) {
            const int off = (16 * (g * JI + h) + sw.n) * SW + 16 * q + 4 * sw.kk;
#pragma unroll
            for (int pl = 0; pl < 3; ++pl) A[h][pl] = lds_bf16x8(&L.S[pl][off]);
        }
    };
    auto state_step = [&](int q, const bf16x8 (&Z)[3]) {
        bf16x8 A[2][JI][3];
        load_group(q, 0, A[0]);
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            if (g + 1 < NG) load_group(q, g + 1, A[(g + 1) & 1]);
            // smallest terms first: (plane, part) = (2,2) (2,1) (1,2) (2,0) (1,1) (0,2) (1,0) (0,1) (0,0)
            constexpr int PL[9] = {2, 2, 1, 2, 1, 0, 1, 0, 0};
            constexpr int PT[9] = {2, 1, 2, 0, 1, 2, 0, 1, 0};
#pragma unroll
            for (int t = 0; t < 9; ++t)
#pragma unroll
                for (int h = 0; h < JI; ++h)
                    YS[g * JI + h] = mfma_bf16x32(A[g & 1][h][PL[t]], Z[PT[t]], YS[g * JI + h]);
        }
    };
    auto apply = [&]() {
        f32x4 Wt[2 * SWv::NS];
#pragma unroll
        for (int ib = 0; ib < 2 * SWv::NS; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r)
                Wt[ib][r] = ib < SWv::NBO
                                ? ((Sp[ib < SWv::NBO ? ib : 0][2][r] + Sp[ib < SWv::NBO ? ib : 0][1][r]) +
                                   Sp[ib < SWv::NBO ? ib : 0][0][r]) * sw.dec[ib][r]
                                : 0.f;
        split_apply<D, C, SWv::NS>(L, Wt, sw.n, sw.kk, YI);
    };
    bf16x8 Za[3], Zb[3];
#pragma unroll
    for (int q = 0; q + 2 < NQ; ++q) {
        split_step(q, Za);
        scores_step(q, Za);
        state_step(q, Za);
    }
    if constexpr (NQ >= 2) {
        split_step(NQ - 2, Za);
        split_step(NQ - 1, Zb);
        scores_step(NQ - 2, Za);
        scores_step(NQ - 1, Zb);
        state_step(NQ - 2, Za);
    } else {
        split_step(0, Zb);
        scores_step(0, Zb);
    }
    apply();
    state_step(NQ - 1, Zb);
}

// ---- staging ----

// bf16 bits of a float that is exactly a bf16 (its high half).
__device__ __forceinline__ uint16_t hi16(float x) { return (uint16_t)(__float_as_uint(x) >> 16); }

// The packed upper block triangle of S^H (as PackedStateRegs holds it:
// thread's group u = 16 bytes of stored block bi, rows 4q..4q+3 of column c
// in accumulator order) written as the three bf16 planes of the full
// symmetric matrix.
template <int D, int NTHR>
__device__ __forceinline__ void stage_state_planes(uint32_t (&S)[3][D * (D / 2 + 8)],
                                                   const PackedStateRegs<D, NTHR>& st, int tid) {
    constexpr int NT = D / 16;
    constexpr int SW = D / 2 + 8;
    constexpr int HPACK = D * (D + 16) / 2;
#pragma unroll
    for (int u = 0; u < PackedStateRegs<D, NTHR>::N; ++u) {
        const int e = (tid + u * NTHR) * 4;
        if (e >= HPACK) continue;
        const int bi = e / 256, l = (e % 256) / 4, q4 = 4 * (l / 16), c = l % 16;
        int a = 0;
#pragma unroll
        for (int aa = 1; aa < NT; ++aa)
            if (bi >= blk_index<NT>(aa, aa)) a = aa;
        const int b = a + (bi - blk_index<NT>(a, a));
        float h[4], m[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float x = st.x[u][r];
            h[r] = __uint_as_float(__float_as_uint(x) & 0xffff0000u);
            const float y = x - h[r];
            m[r] = __uint_as_float(__float_as_uint(y) & 0xffff0000u);
            lo[r] = y - m[r];
        }
        // S[16a + q4 + r][16b + c]
        const int col = perm32(16 * b + c);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * a + q4 + r;
            reinterpret_cast<uint16_t*>(S[0])[row * 2 * SW + col] = hi16(h[r]);
            reinterpret_cast<uint16_t*>(S[1])[row * 2 * SW + col] = hi16(m[r]);
            reinterpret_cast<uint16_t*>(S[2])[row * 2 * SW + col] = hi16(lo[r]);
        }
        // the mirror S[16b + c][16a + q4 + r]: four consecutive permuted columns
        if (a != b) {
            const int w0 = (16 * b + c) * SW + perm32(16 * a + q4) / 2;
            *reinterpret_cast<uint2*>(&S[0][w0]) = make_uint2(pack_hi(h[0], h[1]), pack_hi(h[2], h[3]));
            *reinterpret_cast<uint2*>(&S[1][w0]) = make_uint2(pack_hi(m[0], m[1]), pack_hi(m[2], m[3]));
            *reinterpret_cast<uint2*>(&S[2][w0]) = make_uint2(pack_hi(lo[0], lo[1]), pack_hi(lo[2], lo[3]));
        }
    }
}

// A chunk's bf16 rows as K rows (columns perm32).
template <int D, int C, int NTHR>
__device__ __forceinline__ void stage_key_rows(uint32_t* KR, const ChunkRowsRegs<D, C, NTHR, bf16_t>& rg, int tid) {
    constexpr int SW = D / 2 + 8;
#pragma unroll
    for (int u = 0; u < ChunkRowsRegs<D, C, NTHR, bf16_t>::EL4; ++u) {
        int i, f;
        ChunkRowsRegs<D, C, NTHR, bf16_t>::place(u, tid, i, f);
        *reinterpret_cast<uint2*>(&KR[i * SW + perm32(f) / 2]) = rg.x[u].raw();
    }
}

// A chunk's bf16 rows transposed (feature rows, tokens perm32).
template <int D, int C, int NTHR>
__device__ __forceinline__ void stage_transposed(uint32_t* KT, const ChunkRowsRegs<D, C, NTHR, bf16_t>& rg,
                                                 int tid) {
    constexpr int KW = (C >= 32 ? C : 32) / 2 + 8;
#pragma unroll
    for (int u = 0; u < ChunkRowsRegs<D, C, NTHR, bf16_t>::EL4; ++u) {
        int i, f;
        ChunkRowsRegs<D, C, NTHR, bf16_t>::place(u, tid, i, f);
        const uint2 v = rg.x[u].raw();
        uint16_t* t = reinterpret_cast<uint16_t*>(KT) + perm32(i);
        t[(f + 0) * 2 * KW] = (uint16_t)v.x;
        t[(f + 1) * 2 * KW] = (uint16_t)(v.x >> 16);
        t[(f + 2) * 2 * KW] = (uint16_t)v.y;
        t[(f + 3) * 2 * KW] = (uint16_t)(v.y >> 16);
    }
}

}  // namespace mesa
