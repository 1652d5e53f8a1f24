// cg_h2.h -- the forward CG kernel's chunk machinery with every matvec
// product on fp16 MFMAs over two-part splits (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section "A Camada
// Mesa", bullet "Paralelizacao": the CG over all time steps is a gated-
// linear-attention pass run chunk-parallel on the states.  For chunk c
// (tokens t0..t0+C-1, l_t the within-chunk prefix sum of ln gamma,
// S = S^H_c = H_{t0-1}):
//   H_t p = e^{l_t} S p + sum_{i=t0..t} e^{l_t - l_i} (k_i . p) k_i
//
// Two-part fp16 splits.  A float x is first scaled by a power of two 2^E
// (exact), chosen so that the largest magnitude of the group it belongs to
// lands in [2^14, 2^15); then hi = fp16(x 2^E) and lo = fp16(x 2^E - hi),
// both rounded to nearest.  x 2^E - hi is exact in float and |lo - (x 2^E -
// hi)| <= 2^-11 |x 2^E - hi| <= 2^-22 |x 2^E|, so hi + lo is x 2^E to 22
// bits.  A product a b is then taken as hi_a hi_b + hi_a lo_b + lo_a hi_b
// (three fp16 MFMAs; the dropped lo_a lo_b is below 2^-22 |a b|), so every
// product term carries at most about 3 2^-22 relative error and the sums run
// in fp32.  Magnitudes far below a group's largest fall into fp16's
// subnormal range and keep an absolute error near 2^-25 2^-E: below 2^-39 of
// the group's largest element.  Keys stored as bf16 (8 significant bits) are
// exact in one fp16 part after scaling, so their products take two MFMAs.
//
// Groups and their scales: the chunk state S (one exponent per chunk, from
// max |S_ij|, which for a positive semidefinite S is its largest diagonal
// entry), the chunk's keys and its values (one exponent each per chunk), a
// token's CG direction p and its decayed scores (one exponent per token and
// matvec).  The products' exponents are undone when the fp32 accumulators
// are combined.
//
// LDS layout: a 32-slot MFMA operand of lane group kk is the 4-element
// pieces 4kk..4kk+3 of two 16-column blocks (what the CG vectors hold in
// registers).  Rows of the state planes and key tiles store each 32-column
// block permuted (perm32) so that those eight columns are contiguous: a
// lane's operand is one 128-bit read.  Row pitches are 8 words more than the
// row (an odd multiple of 8 words), so the 16-byte pieces that rows
// m = 0..7 and lane groups kk = 0, 1 read fall on distinct banks.
#pragma once
#include "cg_core.h"
#include "persistent.h"

namespace mesa {

// Position of column c within its 32-column block after the permutation.
__host__ __device__ constexpr int perm32(int c) {
    return 32 * (c / 32) + 8 * ((c % 16) / 4) + 4 * ((c % 32) / 16) + (c % 4);
}

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma_f16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Exponent E with amax 2^E in [2^14, 2^15) (amax > 0), clamped so that 2^E
// and 2^-E are normal floats; 15 for amax = 0.
__device__ __forceinline__ int h2_exp(float amax) {
    const int e = __builtin_amdgcn_frexp_expf(amax);   // amax = f 2^e, f in [0.5, 1)
    return min(max(15 - e, -126), 126);
}
__device__ __forceinline__ float pow2(int e) { return __builtin_amdgcn_ldexpf(1.0f, e); }

// Largest magnitude over the four k-slot lanes n, n+16, n+32, n+48 (the
// lanes of one token); every lane gets the same value.
__device__ __forceinline__ float kslot_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Largest value over all 64 lanes, with lane permutes only (no LDS): within
// each row of 16 lanes over pairs and quads (DPP quad_perm [1,0,3,2] and
// [2,3,0,1]), halves (row_half_mirror) and the row (row_mirror), then across
// the four rows as kslot_max.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_f32<0xb1>(v));
    v = fmaxf(v, dpp_f32<0x4e>(v));
    v = fmaxf(v, dpp_f32<0x141>(v));
    v = fmaxf(v, dpp_f32<0x140>(v));
    return kslot_max(v);
}

template <int N>
__device__ __forceinline__ float absmax(const f32x4 (&A)[N]) {
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(A[j][r]));
    return m;
}

// The two fp16 parts of two 4-element float pieces scaled by s (a power of two).
__device__ __forceinline__ void h2_split(const f32x4& a, const f32x4& b, float s, f16x8& H, f16x8& L) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float y = (e < 4 ? a[e] : b[e - 4]) * s;
        const _Float16 h = (_Float16)y;
        H[e] = h;
        L[e] = (_Float16)(y - (float)h);
    }
}

// The same with a scale per 4-element piece (sa for a, sb for b).
__device__ __forceinline__ void h2_split2(const f32x4& a, const f32x4& b, float sa, float sb, f16x8& H, f16x8& L) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float y = e < 4 ? a[e] * sa : b[e - 4] * sb;
        const _Float16 h = (_Float16)y;
        H[e] = h;
        L[e] = (_Float16)(y - (float)h);
    }
}

// h2_split's result, bit for bit (up to the sign of a zero hi part), at two
// instructions per element: v_fma_mixlo/hi_f16 round s x (exact: s is a
// power of two) to fp16 into the low or high half of the packed hi word, and
// round s x - hi, formed exactly by the same fused operation with hi read
// back from its half, into lo's.  The compiler forms hi twice for h2_split
// (once for the pack, once for the residual), 3.5 instructions per element.
// Inline asm is opaque to the compiler's hazard bookkeeping, so the block
// ends with the two wait states an MFMA reading a VALU result needs; its
// inputs must be VALU results, never an MFMA's (codegen_check.py checks
// both in the built assembly).
__device__ __forceinline__ void h2_split_mix(const f32x4& a, const f32x4& b, float s, f16x8& H, f16x8& L) {
    uint32_t h0, h1, h2, h3, l0, l1, l2, l3;
    asm("v_fma_mixlo_f16 %0, %8, %9, 0\n\t"
        "v_fma_mixhi_f16 %0, %8, %10, 0\n\t"
        "v_fma_mixlo_f16 %1, %8, %11, 0\n\t"
        "v_fma_mixhi_f16 %1, %8, %12, 0\n\t"
        "v_fma_mixlo_f16 %2, %8, %13, 0\n\t"
        "v_fma_mixhi_f16 %2, %8, %14, 0\n\t"
        "v_fma_mixlo_f16 %3, %8, %15, 0\n\t"
        "v_fma_mixhi_f16 %3, %8, %16, 0\n\t"
        "v_fma_mixlo_f16 %4, %8, %9, -%0 op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %4, %8, %10, -%0 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixlo_f16 %5, %8, %11, -%1 op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %5, %8, %12, -%1 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixlo_f16 %6, %8, %13, -%2 op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %6, %8, %14, -%2 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixlo_f16 %7, %8, %15, -%3 op_sel_hi:[0,0,1]\n\t"
        "v_fma_mixhi_f16 %7, %8, %16, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
        "s_nop 1"
        : "=&v"(h0), "=&v"(h1), "=&v"(h2), "=&v"(h3), "=&v"(l0), "=&v"(l1), "=&v"(l2), "=&v"(l3)
        : "v"(s), "v"(a[0]), "v"(a[1]), "v"(a[2]), "v"(a[3]), "v"(b[0]), "v"(b[1]), "v"(b[2]), "v"(b[3]));
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    H = __builtin_bit_cast(f16x8, u32x4{h0, h1, h2, h3});
    L = __builtin_bit_cast(f16x8, u32x4{l0, l1, l2, l3});
}

__device__ __forceinline__ f16x8 lds_f16x8(const uint32_t* p) {
    return __builtin_bit_cast(f16x8, *reinterpret_cast<const uint4*>(p));
}

// Key planes: one (keys stored as bf16, exact in fp16 once scaled) or two.
template <typename In>
__host__ __device__ constexpr int h2_key_planes() { return sizeof(In) == 2 ? 1 : 2; }

// Whether the CG kernel's waves 2 and 3 start their state term from the
// mid-chunk state (d = 128, 64-token chunks, one key plane: the LDS has room
// for its lo plane beside the chunk state's two).  Their intra-chunk terms
// then cover two key blocks at most, as wave 1's, instead of four.
template <int D, int C, int NKP>
__host__ __device__ constexpr bool h2_mid_state() { return D == 128 && C == 64 && NKP == 1; }

template <int D, int C, int NKP>
struct alignas(16) H2Lds {
    static constexpr int SW = D / 2 + 8;                    // words per state / key row
    static constexpr int KW = (C >= 32 ? C : 32) / 2 + 8;   // words per K^T row (at least one 32-key step)
    uint32_t S[2][D * SW];     // S^H_c 2^ES: fp16 planes hi, lo; row r = feature r, columns perm32
    uint32_t KR[NKP][C * SW];  // K_c rows 2^EK, after the CG V_c rows 2^EV (fp16 parts, columns perm32)
    uint32_t KT[NKP][D * KW];  // K_c^T 2^EK (fp16 parts, tokens perm32)
    float L[C];                // l_i
    float Lam[D];
    float red[3][4];           // per-wave maxima: chunk state, keys, values
    int gexp[D / 16];          // exponents of G_c's row blocks while its planes take the state's place
    int next;                  // the claimed next chunk
    // the counters of the mid-chunk state's hand-off between the waves (in
    // what would be the struct's tail padding: the layout stays as without)
    uint32_t hand[h2_mid_state<D, C, NKP>() ? 2 : 1];
};

// Per-wave constants of wave W, for intra-chunk terms over the keys from
// key block KB0 on (an even block: 0, or 2 when the wave's state term starts
// from the mid-chunk state, the state after token 16 KB0 - 1).
template <int D, int C, int W, int KB0 = 0>
struct H2Wave {
    static_assert(KB0 % 2 == 0 && KB0 <= W, "first key block");
    static constexpr int NBO = W + 1 - KB0;    // causal key blocks from block KB0
    static constexpr int NS = (NBO + 1) / 2;   // 32-key steps of the intra-chunk apply
    int n, kk, tr;
    float eLo;                 // e^{l_t - l_{16 KB0 - 1}} (e^{l_t} for KB0 = 0)
    float dec[2 * NS][4];      // e^{l_t - l_i}, key i = 16 (KB0 + ib) + 4kk + r <= t, else 0
    __device__ __forceinline__ H2Wave(const float* Lv, int lane) {
        n = lane & 15;
        kk = lane >> 4;
        tr = 16 * W + n;
        eLo = __expf(KB0 ? Lv[tr] - Lv[16 * KB0 - 1] : Lv[tr]);
#pragma unroll
        for (int ib = 0; ib < 2 * NS; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * (KB0 + ib) + 4 * kk + r;
                dec[ib][r] = (i <= tr) ? __expf(Lv[tr] - Lv[i < C ? i : C - 1]) : 0.f;
            }
    }
};

// Transposed 8-byte LDS read (ds_read_b64_tr_b16): within each group of 16
// lanes, result lane i gets, as element e, half i % 4 of the 8 bytes that
// lane 4 e + i / 4 addresses (the lane layout was checked with a probe).  So
// when lane L of a group addresses row r0 + L / 4 of a row tile, at the
// 4-half piece of columns c0 + 4 (L % 4) .. + 3, lane n receives column
// c0 + n of rows r0 .. r0 + 3.
__device__ __forceinline__ f16x4 lds_tr_f16x4(const uint32_t* p) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef s16x4 __attribute__((address_space(3))) lds_s16x4;
    return __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p)));
}

// The A operand of K^T row block j, 32-key step s, plane pl; the second 16
// keys are zero when the chunk has no such block (C = 16).
template <int D, int C, int NKP>
__device__ __forceinline__ f16x8 h2_kt_operand(const H2Lds<D, C, NKP>& L, int pl, int j, int s, int m, int kk) {
    constexpr int KW = H2Lds<D, C, NKP>::KW;
    if constexpr (C >= 32) {
        return lds_f16x8(&L.KT[pl][(16 * j + m) * KW + 16 * s + 4 * kk]);
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(&L.KT[pl][(16 * j + m) * KW + 4 * kk]);
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        return __builtin_bit_cast(f16x8, u32x4{v.x, v.y, 0u, 0u});
    }
}

// The A operand of V^T row block j (features 16 j + m), 32-token step s,
// plane pl, read transposed from the value rows staged where the key rows
// were: k-slots 8 kk .. 8 kk + 3 are tokens 32 s + 4 kk + e, k-slots 8 kk + 4
// .. 8 kk + 7 tokens 32 s + 16 + 4 kk + e (the order of the B operand's
// decayed scores, and of the tokens in K^T's rows); the second 16 tokens are
// zero when the chunk has no such block (C = 16).
template <int D, int C, int NKP>
__device__ __forceinline__ f16x8 h2_vt_operand(const H2Lds<D, C, NKP>& L, int pl, int j, int s, int m, int kk) {
    constexpr int SW = H2Lds<D, C, NKP>::SW;
    const uint32_t* R = L.KR[pl] + perm32(16 * j + 4 * (m & 3)) / 2;
    const f16x4 a = lds_tr_f16x4(R + (32 * s + 4 * kk + (m >> 2)) * SW);
    const f16x4 b = C >= 32 ? lds_tr_f16x4(R + (32 * s + 16 + 4 * kk + (m >> 2)) * SW) : f16x4{0, 0, 0, 0};
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// Accumulators per key block for the scores: one when several key blocks
// interleave (consecutive MFMAs then never share one), else one per product
// part, summed by h2_score.
template <int NB, int NKP>
__host__ __device__ constexpr int h2_score_parts() { return NB == 1 ? 1 + NKP : 1; }

// Scores of the wave's tokens with key block KB0 + ib (ib < NB), Sc = K Z^T
// 2^(EK + EZ), from the split of Z per 32-feature step.
template <int D, int C, int NKP, int NB, int KB0 = 0>
__device__ __forceinline__ void h2_scores_step(const H2Lds<D, C, NKP>& L, int q, const f16x8& Zh, const f16x8& Zl,
                                               int m, int kk, f32x4 (&Sc)[NB][h2_score_parts<NB, NKP>()]) {
    constexpr int SW = H2Lds<D, C, NKP>::SW;
    constexpr int NP = h2_score_parts<NB, NKP>();
    f16x8 A[NB][NKP];
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
#pragma unroll
        for (int pl = 0; pl < NKP; ++pl)
            A[ib][pl] = lds_f16x8(&L.KR[pl][(16 * (KB0 + ib) + m) * SW + 16 * q + 4 * kk]);
    // smallest terms first
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) Sc[ib][0] = mfma_f16x32(A[ib][0], Zl, Sc[ib][0]);
    if constexpr (NKP == 2) {
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) Sc[ib][NP - 1] = mfma_f16x32(A[ib][1], Zh, Sc[ib][NP - 1]);
    }
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) Sc[ib][NP > 1 ? 1 : 0] = mfma_f16x32(A[ib][0], Zh, Sc[ib][NP > 1 ? 1 : 0]);
}

// Element r of key block ib's scores.
template <int NB, int NKP>
__device__ __forceinline__ float h2_score(const f32x4 (&Sc)[NB][h2_score_parts<NB, NKP>()], int ib, int r) {
    constexpr int NP = h2_score_parts<NB, NKP>();
    if constexpr (NP == 1) return Sc[ib][0][r];
    else if constexpr (NP == 2) return Sc[ib][0][r] + Sc[ib][1][r];
    else return (Sc[ib][0][r] + Sc[ib][2][r]) + Sc[ib][1][r];
}

// Y[j] += V^T row block j (from the value rows) times the decayed scores W over NS 32-key
// steps; W is split here with the per-token exponent EW (W 2^EW):
// Y = T W 2^(ET + EW).
template <int D, int C, int NKP, int NS>
__device__ __forceinline__ void h2_apply(const H2Lds<D, C, NKP>& L, const f32x4 (&W)[2 * NS], float sW, int m,
                                         int kk, f32x4 (&Y)[D / 16]) {
    constexpr int NT = D / 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        f16x8 Wh, Wl;
        h2_split(W[2 * s], W[2 * s + 1], sW, Wh, Wl);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const f16x8 A0 = h2_vt_operand<D, C, NKP>(L, 0, j, s, m, kk);
            Y[j] = mfma_f16x32(A0, Wl, Y[j]);
            if constexpr (NKP == 2) Y[j] = mfma_f16x32(h2_vt_operand<D, C, NKP>(L, 1, j, s, m, kk), Wh, Y[j]);
            Y[j] = mfma_f16x32(A0, Wh, Y[j]);
        }
    }
}

// Y[j] += K^T row block j times the decayed scores W over NS 32-key steps;
// W is split here with the per-token exponent EW (W 2^EW): Y = K^T W 2^(EK + EW).
template <int D, int C, int NKP, int NS>
__device__ __forceinline__ void h2_apply_kt(const H2Lds<D, C, NKP>& L, const f32x4 (&W)[2 * NS], float sW, int m,
                                            int kk, f32x4 (&Y)[D / 16]) {
    constexpr int NT = D / 16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
        f16x8 Wh, Wl;
        h2_split(W[2 * s], W[2 * s + 1], sW, Wh, Wl);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const f16x8 A0 = h2_kt_operand<D, C, NKP>(L, 0, j, s, m, kk);
            Y[j] = mfma_f16x32(A0, Wl, Y[j]);
            if constexpr (NKP == 2) Y[j] = mfma_f16x32(h2_kt_operand<D, C, NKP>(L, 1, j, s, m, kk), Wh, Y[j]);
            Y[j] = mfma_f16x32(A0, Wh, Y[j]);
        }
    }
}

// Y = H_t p for the wave's 16 tokens (no Lambda term), the CG loop's matvec
// as one plain pass: per 32-feature step the split of p (exponent from
// max |p| per token), its scores with the causal keys and its state
// products; then the decayed scores, split, through K^T; then the exponents
// undone in the combination e^{l_t} S p + intra.
template <int D, int C, int NKP, int W>
__device__ __forceinline__ void h2_matvec(const H2Lds<D, C, NKP>& L, const H2Wave<D, C, W>& wv, int ES, int EK,
                                          const f32x4 (&P)[D / 16], f32x4 (&Y)[D / 16]) {
    using Wv = H2Wave<D, C, W>;
    constexpr int NT = D / 16;
    constexpr int NQ = D / 32;
    constexpr int NB = Wv::NBO;
    constexpr int NS = Wv::NS;
    constexpr int NP = h2_score_parts<NB, NKP>();
    constexpr int SW = H2Lds<D, C, NKP>::SW;
    const int n = wv.n, kk = wv.kk;
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    const int EP = h2_exp(kslot_max(absmax<NT>(P)));
    const float sP = pow2(EP);
    f32x4 Sc[NB][NP], YS[NT], YI[NT];
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
#pragma unroll
        for (int t = 0; t < NP; ++t) Sc[ib][t] = zero;
#pragma unroll
    for (int j = 0; j < NT; ++j) YS[j] = YI[j] = zero;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        f16x8 Zh, Zl;
        h2_split(P[2 * q], P[2 * q + 1], sP, Zh, Zl);
        h2_scores_step<D, C, NKP, NB>(L, q, Zh, Zl, n, kk, Sc);
#pragma unroll
        for (int i = 0; i < NT; ++i) {
            const int off = (16 * i + n) * SW + 16 * q + 4 * kk;
            const f16x8 Ah = lds_f16x8(&L.S[0][off]), Al = lds_f16x8(&L.S[1][off]);
            // smallest terms first
            YS[i] = mfma_f16x32(Al, Zh, YS[i]);
            YS[i] = mfma_f16x32(Ah, Zl, YS[i]);
            YS[i] = mfma_f16x32(Ah, Zh, YS[i]);
        }
    }
    f32x4 Wt[2 * NS];
#pragma unroll
    for (int ib = 0; ib < 2 * NS; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Wt[ib][r] = ib < NB ? h2_score<NB, NKP>(Sc, ib < NB ? ib : 0, r) * wv.dec[ib][r] : 0.f;
    const int EW = h2_exp(kslot_max(absmax<2 * NS>(Wt)));
    h2_apply_kt<D, C, NKP, NS>(L, Wt, pow2(EW), n, kk, YI);
    const float a = __builtin_amdgcn_ldexpf(wv.eLo, -(ES + EP));
    const float b = pow2(-(2 * EK + EP + EW));
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) Y[j][r] = a * YS[j][r] + b * YI[j][r];
}

// The CG of wave W on (H_t + Lambda) x = b for its 16 tokens, from x = 0,
// with every matvec on the split products above.  R holds b on entry (B
// layout), X receives the solution; the stop rules are cg_solve's
// (cg_core.h), and so is the arithmetic of x, r and p element for element.
//
// The loop is pipelined so that its vector work runs under the MFMAs:
//  - an iteration forms the new direction p = r + beta p (after the
//    deferred x += alpha p of the previous iteration) one 32-feature step at
//    a time, splits that step and issues its scores and state products
//    before forming the next;
//  - p's exponent therefore cannot wait for max |p|: it comes from the bound
//    b' = |r|_2 + beta b (b = |q|_2 at the start), which bounds |p|_2 and so
//    every element of the new p (up to one rounding): the split never
//    overflows, and while the residuals shrink b' stays within a small
//    factor of |p|_2, which spends a few of fp16's bits of headroom;
//  - the state planes of the next four row blocks are read while the current
//    ones' products run; with bf16 keys (one key plane) the hi plane of the
//    state stays in registers for the whole solve instead (128 words per lane
//    at d = 128, held in accumulator registers, which MFMAs read directly),
//    and only the lo plane is read per iteration;
//  - the apply runs row block by row block, and each block's combination
//    e^{l_t} S p + intra + lambda p and its share of p.Ap follow its MFMAs;
//    the K^T operands are read two row blocks ahead with bf16 keys, one with
//    fp32 keys (the first under the last state products), so their LDS
//    latency does not stall the chain.
// The state term's planes: the hi plane is L.S[0] (read into registers at
// the start with bf16 keys: the chunk state's, or the mid-chunk state's once
// the waves that form it have written it there), or with HI_GIVEN the
// registers SHin the caller filled; the lo plane is Slo (L.S[1], or the
// mid-chunk state's plane); both scaled by 2^ES.  The intra-chunk terms run
// over the causal keys from key block KB0.
template <int D, int NKP>
using H2Hi = f16x8[NKP == 1 ? D / 32 : 1][NKP == 1 ? D / 16 : 1];

// Hand-off between the waves of one workgroup through a counter in LDS,
// without a workgroup barrier: a wave adds one once its earlier LDS reads
// have returned and its LDS writes are done (release), and a wave waits until
// the counter reaches a target (acquire).  The wait gives up after 2^20 polls
// (tens of milliseconds), so that every wave exits even if a count went
// missing.
__device__ __forceinline__ void lds_signal(uint32_t* c, bool leader) {
    if (leader) __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_wait_count(uint32_t* c, uint32_t target) {
    for (int i = 0; i < (1 << 20); ++i) {
        const uint32_t v = __hip_atomic_load(c, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
        if (__builtin_amdgcn_readfirstlane(v) >= target) break;
        __builtin_amdgcn_s_sleep(1);
    }
}

template <int D, int C, int NKP, int W, int KB0, bool HI_GIVEN>
__device__ __forceinline__ int h2_cg_solve(const H2Lds<D, C, NKP>& L, const H2Wave<D, C, W, KB0>& wv, int ES, int EK,
                                           f32x4 (&R)[D / 16], f32x4 (&X)[D / 16], const f32x4 (&lam)[D / 16],
                                           int max_iters, float tol, const uint32_t* Slo, H2Hi<D, NKP>& SHin) {
    using Wv = H2Wave<D, C, W, KB0>;
    constexpr int NT = D / 16;
    constexpr int NQ = D / 32;
    constexpr int NB = Wv::NBO;
    constexpr int NS = Wv::NS;
    constexpr int SW = H2Lds<D, C, NKP>::SW;
    constexpr int JI = NT >= 4 ? 4 : NT;   // row blocks per group of state products
    constexpr int NG = NT / JI;            // groups per 32-feature step
    const int n = wv.n, kk = wv.kk;
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};

    f32x4 P[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        P[j] = R[j];
        X[j] = zero;
    }
    float rr = token_dot<NT>(R, R);
    const float tq = tol * sqrtf(rr);
    const float stop_rr = tq * tq;
    bool done = !(rr > 0.f);   // b == 0 (or a padded token): x = 0, 0 iterations
    int it = 0;
    float alpha = 0.f, beta = 0.f;   // of the previous iteration
    float pbound = sqrtf(rr);        // bounds |p|_2, hence max |p|, of the next direction

    // The hi plane held in registers (bf16 keys: the fp32-key kernel needs
    // those registers for its second key plane, and is slower with it).
    constexpr bool SREG = NKP == 1;
    static_assert(SREG || !HI_GIVEN, "given hi planes need one key plane");
    // a local array (a reference to the caller's makes the compiler hold it
    // worse), copied from the caller's registers or read from L.S[0]
    f16x8 SHr[SREG ? NQ : 1][SREG ? NT : 1];
    if constexpr (SREG) {
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int i = 0; i < NT; ++i)
                SHr[q][i] = HI_GIVEN ? SHin[q][i] : lds_f16x8(&L.S[0][(16 * i + n) * SW + 16 * q + 4 * kk]);
    }
    auto load_group = [&](int f, f16x8 (&A)[JI][2]) {
        const int q = f / NG, g = f % NG;
#pragma unroll
        for (int h = 0; h < JI; ++h) {
            const int off = (16 * (g * JI + h) + n) * SW + 16 * q + 4 * kk;
            if constexpr (!SREG) A[h][0] = lds_f16x8(&L.S[0][off]);
            A[h][1] = lds_f16x8(&Slo[off]);
        }
    };
    auto load_kt = [&](int j, f16x8 (&A)[Wv::NS][NKP]) {
#pragma unroll
        for (int s = 0; s < Wv::NS; ++s)
#pragma unroll
            for (int pl = 0; pl < NKP; ++pl) A[s][pl] = h2_kt_operand<D, C, NKP>(L, pl, j, KB0 / 2 + s, n, kk);
    };

    for (int itn = 0; itn < max_iters; ++itn) {
        if (!done && (rr < stop_rr || rr == 0.f)) done = true;
        if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
        if constexpr (SREG) {
            // keeps the hi plane in accumulator registers (no instruction)
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int i = 0; i < NT; ++i) asm volatile("" : "+a"(SHr[q][i]));
        }
        const int EP = h2_exp(pbound);
        const float sP = pow2(EP);
        constexpr int NP = h2_score_parts<NB, NKP>();
        f32x4 Sc[NB][NP], YS[NT];
#pragma unroll
        for (int ib = 0; ib < NB; ++ib)
#pragma unroll
            for (int t = 0; t < NP; ++t) Sc[ib][t] = zero;
#pragma unroll
        for (int j = 0; j < NT; ++j) YS[j] = zero;
        // the direction's features 32q .. 32q + 31, after the deferred x
        // update, and their split (with fp32 keys the plain split: there the
        // asm block's eight fixed result registers make the compiler move
        // operands through accumulator registers that MFMAs still read)
        f16x8 Z[NQ][2];
        auto form = [&](int q) {
#pragma unroll
            for (int jj = 2 * q; jj < 2 * q + 2; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    X[jj][r] += alpha * P[jj][r];
                    P[jj][r] = R[jj][r] + beta * P[jj][r];
                }
            if constexpr (NKP == 1) h2_split_mix(P[2 * q], P[2 * q + 1], sP, Z[q][0], Z[q][1]);
            else h2_split(P[2 * q], P[2 * q + 1], sP, Z[q][0], Z[q][1]);
        };
        // decayed scores W 2^(EK + EP), their per-token exponent and split
        f16x8 Wh[NS], Wl[NS];
        int EW = 0;
        auto decayed_scores = [&]() {
            f32x4 Wt[2 * NS];
#pragma unroll
            for (int ib = 0; ib < 2 * NS; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    Wt[ib][r] = ib < NB ? h2_score<NB, NKP>(Sc, ib < NB ? ib : 0, r) * wv.dec[ib][r] : 0.f;
            EW = h2_exp(kslot_max(absmax<2 * NS>(Wt)));
            const float sW = pow2(EW);
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                if constexpr (NKP == 1) h2_split_mix(Wt[2 * s], Wt[2 * s + 1], sW, Wh[s], Wl[s]);
                else h2_split(Wt[2 * s], Wt[2 * s + 1], sW, Wh[s], Wl[s]);
            }
        };
        f16x8 SA[2][JI][2];
        // K^T operands of row blocks j .. j + KPF (fp32 keys: two planes, one
        // block ahead, which keeps the ring out of the accumulator registers;
        // 16-token chunks, whose operands are half zeros, read in place)
        constexpr int KPF = C < 32 ? 0 : NKP == 1 ? 2 : 1;
        f16x8 KA[KPF + 1][NS][NKP];
        load_group(0, SA[0]);
        form(0);
        // Per step q: the scores, then the state products, with the next
        // step's direction (or, after the last scores, the decayed scores)
        // formed between the first row group's products and the rest.
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            h2_scores_step<D, C, NKP, NB, KB0>(L, q, Z[q][0], Z[q][1], n, kk, Sc);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int f = q * NG + g;
                if (f + 1 < NQ * NG) {
                    load_group(f + 1, SA[(f + 1) & 1]);
                } else {
                    if constexpr (KPF > 0) load_kt(0, KA[0]);
                    if constexpr (KPF > 1 && NT > 1) load_kt(1, KA[1]);
                }
                const f16x8(&A)[JI][2] = SA[f & 1];
                auto hi = [&](int h) -> const f16x8& {
                    if constexpr (SREG) return SHr[q][g * JI + h];
                    else return A[h][0];
                };
                // smallest terms first
#pragma unroll
                for (int h = 0; h < JI; ++h) YS[g * JI + h] = mfma_f16x32(A[h][1], Z[q][0], YS[g * JI + h]);
#pragma unroll
                for (int h = 0; h < JI; ++h) YS[g * JI + h] = mfma_f16x32(hi(h), Z[q][1], YS[g * JI + h]);
#pragma unroll
                for (int h = 0; h < JI; ++h) YS[g * JI + h] = mfma_f16x32(hi(h), Z[q][0], YS[g * JI + h]);
                if (g == 0) {
                    if (q + 1 < NQ) form(q + 1);
                    else decayed_scores();
                }
            }
        }
        const float a = __builtin_amdgcn_ldexpf(wv.eLo, -(ES + EP));
        const float b = pow2(-(2 * EK + EP + EW));
        // apply, combination and p.Ap, one row block at a time
        f32x4 Y[NT];
        float pp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (j + KPF < NT) load_kt(j + KPF, KA[(j + KPF) % (KPF + 1)]);
            const f16x8(&KJ)[NS][NKP] = KA[j % (KPF + 1)];
            f32x4 yi = zero;
#pragma unroll
            for (int s = 0; s < NS; ++s) {
                yi = mfma_f16x32(KJ[s][0], Wl[s], yi);
                if constexpr (NKP == 2) yi = mfma_f16x32(KJ[s][1], Wh[s], yi);
                yi = mfma_f16x32(KJ[s][0], Wh[s], yi);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Y[j][r] = a * YS[j][r] + (b * yi[r] + lam[j][r] * P[j][r]);
                pp[r] += P[j][r] * Y[j][r];
            }
        }
        const float pap = kslot_sum((pp[0] + pp[1]) + (pp[2] + pp[3]));
        const bool act = !done && (pap > 0.f);
        if (!done && !act) done = true;   // breakdown guard
        alpha = act ? rcp_div(rr, pap) : 0.f;
        float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                R[j][r] -= alpha * Y[j][r];
                rs[r] += R[j][r] * R[j][r];
            }
        const float rrn = kslot_sum((rs[0] + rs[1]) + (rs[2] + rs[3]));
        // a stopped token gets beta = 0: its direction becomes its frozen residual
        beta = act ? rcp_div(rrn, rr) : 0.f;
        pbound = sqrtf(rrn) + beta * pbound;
        rr = act ? rrn : rr;
        it += act ? 1 : 0;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) X[j][r] += alpha * P[j][r];
    return it;
}

// The mid-chunk state S_m = e^{l_{M-1}} S + sum_{i<M} e^{l_{M-1} - l_i} k_i k_i^T
// (M = 16 KB0 tokens: the state after the chunk's first M tokens), formed by
// a share of the waves: the operand pieces (q, i) (32-feature step q, row
// block i) numbered q D/16 + i in [PB, PE), their hi parts into the wave's
// registers SHr[q][i], their lo parts into Slo (laid out as L.S's planes);
// returns the planes' exponent (they hold S_m 2^E), which every wave that
// forms a share computes alike.
//  - Tile (c, i) of S_m (rows 16c.., columns 16i..) is e^{l_{M-1}} times S's
//    tile plus the weighted keys' row block c times the keys' row block i,
//    over the M keys, on fp16 MFMAs: the keys are exact in one fp16 part, the
//    weighted keys take two (hi, lo).  In the accumulator layout lane (n, kk)
//    holds rows 16c + 4kk + r of column 16i + n, which by symmetry is row
//    16i + n at columns 16c + 4kk + r: tiles (2q, i) and (2q + 1, i) together
//    are the operand piece (q, i) of row block i, and S's part of them is the
//    piece its planes hold at row 16i + n (added after the MFMAs, which start
//    from zero: an accumulator input written just before would be rewritten
//    for the next tile while the MFMA may still read it).
//  - The accumulators carry 2^EA, EA = 2 EK: the weighted keys then lie in
//    fp16's normal range as the scores' keys do (a smaller EA, e.g. the zero
//    state's default exponent, flushed them to zero for keys far below unit
//    size), and the keys' part stays below 2^35.  EA is capped at ES + 100 so
//    that S's part stays below 2^115; where the cap binds the keys' part is
//    far below S's and may underflow.  One exponent for the whole matrix
//    comes from its largest diagonal entry (a positive semidefinite matrix's
//    largest magnitude), formed first on the VALU.
template <int D, int C, int NKP, int KB0, int PB, int PE>
__device__ __forceinline__ int h2_form_mid(const H2Lds<D, C, NKP>& L, int ES, int EK, int n, int kk, uint32_t* Slo,
                                           H2Hi<D, NKP>& SHr) {
    static_assert(NKP == 1 && KB0 == 2 && C >= 16 * KB0, "one key plane, 32 keys before the mid-chunk state");
    constexpr int NT = D / 16;
    static_assert(0 <= PB && PB < PE && PE <= NT * D / 32, "operand pieces formed");
    constexpr int QB = PB / NT, QE = (PE - 1) / NT + 1;   // their 32-feature steps
    constexpr int SW = H2Lds<D, C, NKP>::SW;
    constexpr int M = 16 * KB0;
    const float lm = L.L[M - 1];
    const int EA = min(2 * EK, ES + 100);
    const float fS = __builtin_amdgcn_ldexpf(__expf(lm), EA - ES);
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    // weights of the lane's 8 key slots (32-key step 0: slot e < 4 is key
    // 4kk + e, slot 4 + e key 16 + 4kk + e), times 2^(EA - 2EK)
    float wsl[8];
#pragma unroll
    for (int e = 0; e < 8; ++e)
        wsl[e] = __builtin_amdgcn_ldexpf(__expf(lm - L.L[(e < 4 ? 0 : 16) + 4 * kk + (e & 3)]), EA - 2 * EK);
    // K^T row blocks over the first 32 keys: the B operand of column block i,
    // and (weighted) the A operand of row block c, of lane (n, kk)
    f16x8 B[NT];
#pragma unroll
    for (int i = 0; i < NT; ++i) B[i] = h2_kt_operand<D, C, NKP>(L, 0, i, 0, n, kk);
    // the weighted keys' row blocks as A operands (those of the pieces
    // formed), split once
    f16x8 Ah[NT], Al[NT];
#pragma unroll
    for (int c = 2 * QB; c < 2 * QE; ++c) {
        f32x4 a, b;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            a[e] = (float)B[c][e] * wsl[e];
            b[e] = (float)B[c][4 + e] * wsl[4 + e];
        }
        h2_split_mix(a, b, 1.0f, Ah[c], Al[c]);
    }
    // a0, a1 plus S's tiles (2q, i) and (2q + 1, i) times e^{l_{M-1}}
    // 2^(EA - ES), on mixed-precision fmas from the fp16 parts
    auto add_s = [&](int i, int q, f32x4& a0, f32x4& a1) {
        const int off = (16 * i + n) * SW + 16 * q + 4 * kk;
        const f16x8 h = lds_f16x8(&L.S[0][off]), l = lds_f16x8(&L.S[1][off]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            a0[r] = fmaf((float)h[r], fS, fmaf((float)l[r], fS, a0[r]));
            a1[r] = fmaf((float)h[4 + r], fS, fmaf((float)l[4 + r], fS, a1[r]));
        }
    };
    // the diagonal, entry 16c + n: S's entry times e^{l_{M-1}} 2^(EA - ES)
    // plus the lane group's weighted squares summed over the four groups (the
    // tiles' own diagonals may differ from it by rounding: the exponent then
    // leaves the largest element within an ulp of the range it aims for)
    float dmax = 0.f;
#pragma unroll
    for (int c = 0; c < NT; ++c) {
        float sq = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) sq = fmaf((float)B[c][e] * wsl[e], (float)B[c][e], sq);
        const int a = 16 * c + n;
        const int pc = perm32(a);
        const uint32_t wh = L.S[0][a * SW + pc / 2], wl = L.S[1][a * SW + pc / 2];
        const _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)(pc & 1 ? wh >> 16 : wh & 0xffff));
        const _Float16 l = __builtin_bit_cast(_Float16, (uint16_t)(pc & 1 ? wl >> 16 : wl & 0xffff));
        dmax = fmaxf(dmax, fabsf(fmaf((float)h + (float)l, fS, kslot_sum(sq))));
    }
    const int EM = h2_exp(wave_max(dmax));
    const float sM = pow2(EM);
#pragma unroll
    for (int q = QB; q < QE; ++q) {
#pragma unroll
        for (int i = (q * NT < PB ? PB - q * NT : 0); i < (PE - q * NT < NT ? PE - q * NT : NT); ++i) {
            f32x4 a0 = mfma_f16x32(Al[2 * q], B[i], zero);
            a0 = mfma_f16x32(Ah[2 * q], B[i], a0);
            f32x4 a1 = mfma_f16x32(Al[2 * q + 1], B[i], zero);
            a1 = mfma_f16x32(Ah[2 * q + 1], B[i], a1);
            add_s(i, q, a0, a1);   // VALU results: the asm split may take them
            f16x8 lo;
            h2_split_mix(a0, a1, sM, SHr[q][i], lo);
            *reinterpret_cast<uint4*>(&Slo[(16 * i + n) * SW + 16 * q + 4 * kk]) = __builtin_bit_cast(uint4, lo);
        }
    }
    return EA + EM;
}

// ---- staging ----

// Largest magnitude this thread holds of the packed upper block triangle.
template <int D, int NTHR>
__device__ __forceinline__ float packed_absmax(const PackedStateRegs<D, NTHR>& st, int tid) {
    float m = 0.f;
#pragma unroll
    for (int u = 0; u < PackedStateRegs<D, NTHR>::N; ++u)
        if ((tid + u * NTHR) * 4 < PackedStateRegs<D, NTHR>::HPACK)
#pragma unroll
            for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(st.x[u][r]));
    return m;
}

// Largest magnitude this thread holds of a chunk's rows.
template <int D, int C, int NTHR, typename In>
__device__ __forceinline__ float rows_absmax(const ChunkRowsRegs<D, C, NTHR, In>& rg) {
    float m = 0.f;
#pragma unroll
    for (int u = 0; u < ChunkRowsRegs<D, C, NTHR, In>::EL4; ++u) {
        const f32x4 v = rg.x[u].get();
#pragma unroll
        for (int r = 0; r < 4; ++r) m = fmaxf(m, fabsf(v[r]));
    }
    return m;
}

// The packed upper block triangle of S^H (PackedStateRegs: the thread's
// group u = 16 bytes of stored block bi, rows 4q..4q+3 of column c in
// accumulator order) scaled by s, written as the two fp16 planes of the full
// symmetric matrix.
template <int D, int NTHR>
__device__ __forceinline__ void stage_h2_state(uint32_t (&S)[2][D * (D / 2 + 8)], const PackedStateRegs<D, NTHR>& st,
                                               int tid, float s) {
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
        _Float16 h[4], lo[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float y = st.x[u][r] * s;
            h[r] = (_Float16)y;
            lo[r] = (_Float16)(y - (float)h[r]);
        }
        // S[16a + q4 + r][16b + c]
        const int col = perm32(16 * b + c);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * a + q4 + r;
            reinterpret_cast<_Float16*>(S[0])[row * 2 * SW + col] = h[r];
            reinterpret_cast<_Float16*>(S[1])[row * 2 * SW + col] = lo[r];
        }
        // the mirror S[16b + c][16a + q4 + r]: four consecutive permuted columns
        if (a != b) {
            const int w0 = (16 * b + c) * SW + perm32(16 * a + q4) / 2;
            *reinterpret_cast<f16x4*>(&S[0][w0]) = f16x4{h[0], h[1], h[2], h[3]};
            *reinterpret_cast<f16x4*>(&S[1][w0]) = f16x4{lo[0], lo[1], lo[2], lo[3]};
        }
    }
}

// A chunk's rows scaled by s as NKP fp16 planes of K rows (columns perm32).
template <int D, int C, int NTHR, int NKP, typename In>
__device__ __forceinline__ void stage_h2_rows(uint32_t (&KR)[NKP][C * (D / 2 + 8)],
                                              const ChunkRowsRegs<D, C, NTHR, In>& rg, int tid, float s) {
    constexpr int SW = D / 2 + 8;
#pragma unroll
    for (int u = 0; u < ChunkRowsRegs<D, C, NTHR, In>::EL4; ++u) {
        int i, f;
        ChunkRowsRegs<D, C, NTHR, In>::place(u, tid, i, f);
        const f32x4 v = rg.x[u].get();
        f16x4 h, lo;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float y = v[r] * s;
            h[r] = (_Float16)y;
            lo[r] = (_Float16)(y - (float)h[r]);
        }
        *reinterpret_cast<f16x4*>(&KR[0][i * SW + perm32(f) / 2]) = h;
        if constexpr (NKP == 2) *reinterpret_cast<f16x4*>(&KR[1][i * SW + perm32(f) / 2]) = lo;
    }
}

// A chunk's rows scaled by s, transposed (feature rows, tokens perm32), as
// NKP fp16 planes.
template <int D, int C, int NTHR, int NKP, typename In>
__device__ __forceinline__ void stage_h2_transposed(uint32_t (&KT)[NKP][D * ((C >= 32 ? C : 32) / 2 + 8)],
                                                    const ChunkRowsRegs<D, C, NTHR, In>& rg, int tid, float s) {
    constexpr int KW = (C >= 32 ? C : 32) / 2 + 8;
#pragma unroll
    for (int u = 0; u < ChunkRowsRegs<D, C, NTHR, In>::EL4; ++u) {
        int i, f;
        ChunkRowsRegs<D, C, NTHR, In>::place(u, tid, i, f);
        const f32x4 v = rg.x[u].get();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float y = v[r] * s;
            const _Float16 h = (_Float16)y;
            reinterpret_cast<_Float16*>(KT[0])[(f + r) * 2 * KW + perm32(i)] = h;
            if constexpr (NKP == 2) reinterpret_cast<_Float16*>(KT[1])[(f + r) * 2 * KW + perm32(i)] = (_Float16)(y - (float)h);
        }
    }
}

// The staging of a chunk, in two steps around a workgroup barrier: each wave
// puts the largest magnitudes of its share of the chunk state and keys in
// L.red; after the barrier every wave takes the chunk's exponents from them
// and writes its share of the state planes, the key rows and K^T.
template <int D, int C, int NTHR, int NKP, typename In>
__device__ __forceinline__ void h2_put_maxima(H2Lds<D, C, NKP>& L, const PackedStateRegs<D, NTHR>& st,
                                              const ChunkRowsRegs<D, C, NTHR, In>& kr, int tid, int lane, int w) {
    const float sm = wave_max(packed_absmax<D, NTHR>(st, tid));
    const float km = wave_max(rows_absmax<D, C, NTHR, In>(kr));
    if (lane == 0) {
        L.red[0][w] = sm;
        L.red[1][w] = km;
    }
}

template <int D, int C, int NTHR, int NKP, typename In>
__device__ __forceinline__ void h2_stage_chunk(H2Lds<D, C, NKP>& L, const PackedStateRegs<D, NTHR>& st,
                                               const ChunkRowsRegs<D, C, NTHR, In>& kr, int tid, int& ES, int& EK) {
    constexpr int NW = NTHR / 64;
    float smax = 0.f, kmax = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) {
        smax = fmaxf(smax, L.red[0][w2]);
        kmax = fmaxf(kmax, L.red[1][w2]);
    }
    ES = __builtin_amdgcn_readfirstlane(h2_exp(smax));
    EK = __builtin_amdgcn_readfirstlane(h2_exp(kmax));
    stage_h2_state<D, NTHR>(L.S, st, tid, pow2(ES));
    stage_h2_rows<D, C, NTHR, NKP, In>(L.KR, kr, tid, pow2(EK));
    stage_h2_transposed<D, C, NTHR, NKP, In>(L.KT, kr, tid, pow2(EK));
}

// The workgroup's first chunk: its state, keys, gates and lambda, staged
// (ends with a barrier).
template <int D, int C, int NTHR, int NKP, typename In>
__device__ __forceinline__ void h2_stage_first(H2Lds<D, C, NKP>& L, const ChunkPos& p, const float* __restrict__ SH,
                                               const In* __restrict__ k, const float* __restrict__ gamma,
                                               const float* __restrict__ lambda, int tid, int& ES, int& EK) {
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    PackedStateRegs<D, NTHR> s0;
    s0.load(SH + p.hoff, tid);
    ChunkRowsRegs<D, C, NTHR, In> k0;
    k0.load(k + p.tok0 * D, p.valid, tid);
    h2_put_maxima<D, C, NTHR, NKP, In>(L, s0, k0, tid, lane, w);
    for (int e = tid; e < D; e += NTHR) L.Lam[e] = lambda[(size_t)p.h * D + e];
    if (w == 0) {
        const float l = chunk_log_decay(gamma + p.tok0, p.valid, lane);
        if (lane < C) L.L[lane] = l;
    }
    __syncthreads();
    h2_stage_chunk<D, C, NTHR, NKP, In>(L, s0, k0, tid, ES, EK);
    __syncthreads();
}

}  // namespace mesa

