// bwd_kv.hip -- the backward's key and value gradients (gfx950).
//
// Implicit differentiation of o_t = G_t (H_t + Lambda)^{-1} q_t (the page,
// section "A Camada Mesa", bullet "Paralelizacao", says the layer trains in
// parallel but gives no gradient), at the forward's solutions x_t and the
// adjoint solutions z_t, for a loss with dL/do_t = g_t:
//   dL/dv_i = sum_{t>=i} zeta_ti (x_t . k_i) g_t
//   dL/dk_i = sum_{t>=i} zeta_ti [(g_t . v_i) x_t - (x_t . k_i) z_t - (z_t . k_i) x_t]
//   a_i     = (v_i . dL/dv_i + k_i . dL/dk_i) / 2      (the key-side gate total)
// Chunkwise, for key i of chunk c (l the within-chunk prefix sums, e_c the
// chunk's last token), the later chunks enter through the reverse states:
//   dv_i = sum_{t in c, t>=i} e^{l_t - l_i} (x_t . k_i) g_t + e^{l_e - l_i} P^gx_c k_i
//   dk_i = sum_{t in c, t>=i} e^{l_t - l_i} [(g_t . v_i - z_t . k_i) x_t - (x_t . k_i) z_t]
//          + e^{l_e - l_i} [(P^gx_c)^T v_i - (P^zx_c + (P^zx_c)^T) k_i]
// Work split: one workgroup per (head, chunk); wave w owns keys 16w..16w+15
// and holds their k_i, v_i in registers as the MFMA B operand (lane (n, kk):
// features 16j + 4kk + r of key n).  The state terms come first: the
// reverse-state kernel stores P^gx and the symmetric M = P^zx + (P^zx)^T
// once each, in accumulator block order, which is the operand order of the
// transpose; so P columns (rows of P^T) and M rows are A operands read
// straight from memory, and P rows come from the same blocks passed through
// a per-wave LDS transpose.  Meanwhile the
// chunk's x, z, g rows travel from memory into LDS by direct loads.  Then
// the within-chunk sums: scores come out of the MFMA in exactly the layout
// the next contraction (over tokens) takes as its B operand, so the token
// tiles are the A operand both ways, read along rows for the scores and
// down columns for the sums over tokens.  Every MFMA chain starts from zero
// and is only read afterwards.
#include "cg_h2.h"
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

// Per-wave scratch of the P block transposes.  d = 16 (fp32 states): one
// block, element (row, col) at (row / 4) * kTrPitch + 4 col + row % 4 (pitch
// 68: the transposed reads hit 64 distinct banks).  d >= 32 (fp16 states):
// one 2 x 2 super-block as rows of P^T, two planes (hi, lo) of 32 rows x 32
// halves, rows kTrRow words apart and rows 8..15 of each 16 shifted by 4
// words (kTrRow = 24: the eight rows a half-wave's transposed read touches
// fall on distinct 8-bank windows; the shift puts the sixteen rows a
// half-wave's writes touch on distinct 4-bank windows).
constexpr int kTrPitch = 68;
constexpr int kTrBlock = 4 * kTrPitch;
constexpr int kTrRow = 24;
constexpr int kTrPlane = 32 * kTrRow;

template <int D, int C>
struct alignas(16) KvLds {
    static constexpr int PD = lds_pitch(D);
    static constexpr int TRW = D >= 32 ? 2 * kTrPlane : (D / 16) * kTrBlock;   // scratch words per wave
    float R[3 * C * PD];   // x, z, g rows of the chunk
    float L[C];
    float Tr[C / 16][TRW];   // per-wave transpose scratch
    // with four waves: the within-chunk sums of key block 0 over token block
    // 3, which wave 3 takes from wave 0: the D / 16 16-byte pieces of dk, then
    // of dv, each piece stored for the 64 lanes in turn (32 D floats)
    float Pk0[C == 64 ? 32 * D : 4];
};

// Whether wave 3 takes key block 0's sums over token block 3 from wave 0
// (four waves: their within-chunk pairs of key and token blocks, 4, 3, 2, 1,
// become 3, 3, 2, 2).
template <int C>
__host__ __device__ constexpr bool kv_rebalance() { return C == 64; }

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Sc[tb] = A[16tb + m][:] . Z^T[:][n]: scores of the chunk's token rows
// (tile rows, pitch lds_pitch(D)) against the wave's keys or values in registers.
template <int D>
__device__ __forceinline__ f32x4 token_scores(const float* rows, const f32x4 (&Z)[D / 16], int m, int kk) {
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    const float* a = rows + m * PD + 4 * kk;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 buf[2];
    buf[0] = ld4(a);
#pragma unroll
    for (int gg = 0; gg < NT; ++gg) {
        if (gg + 1 < NT) buf[(gg + 1) & 1] = ld4(a + 16 * (gg + 1));
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma4(buf[gg & 1][s], Z[gg][s], acc);
    }
    return acc;
}

// The later chunks' terms for the wave's keys, from the stored states (block
// (a, b) of a state at 256 (a NT + b) floats, accumulator order):
//   A1 = P^gx k_i,   A2 = (P^gx)^T v_i - (P^zx + (P^zx)^T) k_i.
// P^gx's block (a, b) is (P^gx)^T's operand block (b, a), so it feeds A2[b]
// with v_i's features of block a as it comes; its transpose is P^gx's operand
// block (a, b), which feeds A1[a] with k_i's features of block b.  The blocks
// go by diagonals (b = a + dg mod NT), so consecutive blocks update different
// accumulators of both sums; a diagonal's blocks are transposed through the
// wave's LDS scratch while the A2 products of the diagonal run.
template <int D>
__device__ __forceinline__ void state_terms(const float* __restrict__ Pg, const float* __restrict__ Pz, int lane,
                                            const f32x4 (&Kb)[D / 16], const f32x4 (&Vb)[D / 16],
                                            f32x4 (&A1)[D / 16], f32x4 (&A2)[D / 16], float* tr) {
    constexpr int NT = D / 16;
    const float* pg = Pg + 4 * lane;
    const float* pz = Pz + 4 * lane;
    const int m = lane & 15, q = lane >> 4;
    f32x4 A3[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) A1[j] = A2[j] = A3[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto ld = [](const float* p) { return *reinterpret_cast<const f32x4*>(p); };
    f32x4 bg[2][NT];
    // diagonal dg: block (a, (a + dg) % NT) for a = 0..NT-1
    auto load_d = [&](int dg, int buf) {
#pragma unroll
        for (int a = 0; a < NT; ++a) bg[buf][a] = ld(pg + (a * NT + (a + dg) % NT) * 256);
    };
    load_d(0, 0);
#pragma unroll
    for (int dg = 0; dg < NT; ++dg) {
        const int cb = dg & 1;
        // the diagonal's blocks into the scratch, in accumulator layout
#pragma unroll
        for (int a = 0; a < NT; ++a) *reinterpret_cast<f32x4*>(tr + a * kTrBlock + q * kTrPitch + 4 * m) = bg[cb][a];
        if (dg + 1 < NT) load_d(dg + 1, cb ^ 1);
        // A2[b] += P^T_op(b, a) v(a)
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int a = 0; a < NT; ++a) {
                const int b = (a + dg) % NT;
                A2[b] = mfma4(bg[cb][a][s], Vb[a][s], A2[b]);
            }
        wave_lds_sync();
        // A1[a] += P_op(a, b) k(b): element u of lane (q, m) is row m, column 4q + u of the block
        f32x4 t[NT];
#pragma unroll
        for (int a = 0; a < NT; ++a)
#pragma unroll
            for (int u = 0; u < 4; ++u) t[a][u] = tr[a * kTrBlock + (m >> 2) * kTrPitch + 4 * (4 * q + u) + (m & 3)];
        wave_lds_sync();
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int a = 0; a < NT; ++a) {
                const int b = (a + dg) % NT;
                A1[a] = mfma4(t[a][s], Kb[b][s], A1[a]);
            }
    }
    // rows of M = P^zx + (P^zx)^T: M's operand-order block (j, g) is its
    // stored accumulator-order block (g, j), M being symmetric
    auto load_z = [&](int g, int buf) {
#pragma unroll
        for (int j = 0; j < NT; ++j) bg[buf][j] = ld(pz + (g * NT + j) * 256);
    };
    load_z(0, 0);
#pragma unroll
    for (int g = 0; g < NT; ++g) {
        if (g + 1 < NT) load_z(g + 1, (g + 1) & 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < NT; ++j) A3[j] = mfma4(bg[g & 1][j][s], Kb[g][s], A3[j]);
    }
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) A2[j][r] -= A3[j][r];
}

// d >= 32: the stored states are two-part fp16 splits (a lane's 16 bytes:
// hi then lo of its four values) with an exponent per stored 16-row block
// (EP for P^gx, EM for M).  P^gx's blocks go by 2 x 2 super-blocks (rows 2A,
// 2A + 1, columns 2B, 2B + 1), diagonal by diagonal: the accumulator-order
// pair (2A, b), (2A + 1, b) is a 32-slot operand of (P^gx)^T for A2[b] as it
// comes; written as rows of P^T into the wave's scratch, the super-block
// comes back through the transposed LDS read as P's operand pairs (a, 2B),
// (a, 2B + 1) for A1[a].  An exponent that varies along a contraction (EP[a]
// for A2, EM[g] for A3) is folded into that operand's split of v or k, so
// every accumulator chain keeps one scale; the scales are undone at the end.
template <int D>
__device__ __forceinline__ void state_terms_h2(const float* __restrict__ Pg, const float* __restrict__ Pz,
                                               const int* __restrict__ Eg, const int* __restrict__ Ez, int lane,
                                               const f32x4 (&Kb)[D / 16], const f32x4 (&Vb)[D / 16],
                                               f32x4 (&A1)[D / 16], f32x4 (&A2)[D / 16], float* trf) {
    constexpr int NT = D / 16;
    constexpr int NP = NT / 2;
    typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
    uint32_t* tr = reinterpret_cast<uint32_t*>(trf);
    const int m = lane & 15, q = lane >> 4;
    int EP[NT], EM[NT];
    int cP = 1 << 30, cM = 1 << 30;
#pragma unroll
    for (int a = 0; a < NT; ++a) {
        EP[a] = Eg[a];
        EM[a] = Ez[a];
        cP = min(cP, EP[a]);
        cM = min(cM, EM[a]);
    }
    // per-key exponents (the B operand's columns are the wave's keys)
    const int EK = h2_exp(kslot_max(absmax<NT>(Kb)));
    const int EV = h2_exp(kslot_max(absmax<NT>(Vb)));
    f16x8 Kh[NP], Kl[NP], Mh[NP], Ml[NP], Vh[NP], Vl[NP];
#pragma unroll
    for (int pp = 0; pp < NP; ++pp) {
        h2_split(Kb[2 * pp], Kb[2 * pp + 1], pow2(EK), Kh[pp], Kl[pp]);
        h2_split2(Kb[2 * pp], Kb[2 * pp + 1], pow2(EK + cM - EM[2 * pp]), pow2(EK + cM - EM[2 * pp + 1]), Mh[pp],
                  Ml[pp]);
        h2_split2(Vb[2 * pp], Vb[2 * pp + 1], pow2(EV + cP - EP[2 * pp]), pow2(EV + cP - EP[2 * pp + 1]), Vh[pp],
                  Vl[pp]);
    }
    const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 A3[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) A1[j] = A2[j] = A3[j] = zero;
    auto ld = [&](const float* P, int a, int b) {
        return *reinterpret_cast<const u32x4v*>(P + (a * NT + b) * 256 + 4 * lane);
    };
    // operand of two stacked blocks' plane pl (0: hi, 1: lo)
    auto pair = [](const u32x4v& u, const u32x4v& v, int pl) {
        typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
        return __builtin_bit_cast(f16x8, pl == 0 ? u32x4s{u[0], u[1], v[0], v[1]} : u32x4s{u[2], u[3], v[2], v[3]});
    };
    u32x4v blk[2][2][2];   // [buffer][i][jb]: block (2A + i, 2B + jb)
    auto load_sb = [&](int s, int buf) {
        const int A = s % NP, B = (A + s / NP) % NP;
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) blk[buf][i][jb] = ld(Pg, 2 * A + i, 2 * B + jb);
    };
    load_sb(0, 0);
#pragma unroll
    for (int s = 0; s < NP * NP; ++s) {
        const int A = s % NP, B = (A + s / NP) % NP, cb = s & 1;
        // the super-block as rows of P^T: row 16 jb + m, words 8 i + 2 q (P rows 16 i + 4 q .. + 3)
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
#pragma unroll
                for (int pl = 0; pl < 2; ++pl)
                    *reinterpret_cast<uint2*>(
                        &tr[pl * kTrPlane + (16 * jb + m) * kTrRow + 4 * (m >> 3) + 8 * i + 2 * q]) =
                        make_uint2(blk[cb][i][jb][2 * pl], blk[cb][i][jb][2 * pl + 1]);
        if (s + 1 < NP * NP) load_sb(s + 1, cb ^ 1);
        // A2[b] += P^T_op(b, 2A..2A+1) v(2A..2A+1)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const f16x8 oh = pair(blk[cb][0][jb], blk[cb][1][jb], 0), ol = pair(blk[cb][0][jb], blk[cb][1][jb], 1);
            f32x4& acc = A2[2 * B + jb];
            acc = mfma_f16x32(ol, Vh[A], acc);
            acc = mfma_f16x32(oh, Vl[A], acc);
            acc = mfma_f16x32(oh, Vh[A], acc);
        }
        wave_lds_sync();
        // A1[a] += P_op(a, 2B..2B+1) k(2B..2B+1): lane (m, q) receives P[16 a + m][16 b + 4 q + e]
        f16x8 op[2][2];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int pl = 0; pl < 2; ++pl) {
                const int row = 4 * q + (m >> 2);   // of 16 (jb = 0; jb = 1 adds 16 rows)
                const uint32_t* base = &tr[pl * kTrPlane + row * kTrRow + 4 * (row >> 3) + 8 * i + 2 * (m & 3)];
                const f16x4 t0 = lds_tr_f16x4(base), t1 = lds_tr_f16x4(base + 16 * kTrRow);
                op[i][pl] = f16x8{t0[0], t0[1], t0[2], t0[3], t1[0], t1[1], t1[2], t1[3]};
            }
        wave_lds_sync();
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            f32x4& acc = A1[2 * A + i];
            acc = mfma_f16x32(op[i][1], Kh[B], acc);
            acc = mfma_f16x32(op[i][0], Kl[B], acc);
            acc = mfma_f16x32(op[i][0], Kh[B], acc);
        }
    }
    // rows of M = P^zx + (P^zx)^T: M's operand-order block (j, g) is its stored
    // accumulator-order block (g, j), M being symmetric
    u32x4v zb[2][2][NT];   // [buffer][g parity][j]
    auto load_z = [&](int G, int buf) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            zb[buf][0][j] = ld(Pz, 2 * G, j);
            zb[buf][1][j] = ld(Pz, 2 * G + 1, j);
        }
    };
    load_z(0, 0);
#pragma unroll
    for (int G = 0; G < NP; ++G) {
        if (G + 1 < NP) load_z(G + 1, (G + 1) & 1);
        const int cb = G & 1;
#pragma unroll
        for (int j = 0; j < NT; ++j) A3[j] = mfma_f16x32(pair(zb[cb][0][j], zb[cb][1][j], 1), Mh[G], A3[j]);
#pragma unroll
        for (int j = 0; j < NT; ++j) A3[j] = mfma_f16x32(pair(zb[cb][0][j], zb[cb][1][j], 0), Ml[G], A3[j]);
#pragma unroll
        for (int j = 0; j < NT; ++j) A3[j] = mfma_f16x32(pair(zb[cb][0][j], zb[cb][1][j], 0), Mh[G], A3[j]);
    }
    const float s2 = pow2(-(EV + cP)), s3 = pow2(-(EK + cM));
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const float s1 = pow2(-(EK + EP[j]));
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            A1[j][r] *= s1;
            A2[j][r] = s2 * A2[j][r] - s3 * A3[j][r];
        }
    }
}

// The within-chunk sums of keys i (lane (n, kk): key il, log decay li, its
// k and v in Kb, Vb) over token block tb (tokens t >= i): BK, BV as fresh MFMA
// chains; the value gradient's weights are the negated x_t . k_i weights of
// the key gradient's.
template <int D>
__device__ __forceinline__ void kv_pair(const float* X, const float* Zt, const float* Gt, const float* Lv, int tb,
                                        const f32x4 (&Kb)[D / 16], const f32x4 (&Vb)[D / 16], int il, float li,
                                        int n, int kk, f32x4 (&BK)[D / 16], f32x4 (&BV)[D / 16]) {
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    const f32x4 s1 = token_scores<D>(X + 16 * tb * PD, Kb, n, kk);    // x_t . k_i
    const f32x4 s2 = token_scores<D>(Gt + 16 * tb * PD, Vb, n, kk);   // g_t . v_i
    const f32x4 s3 = token_scores<D>(Zt + 16 * tb * PD, Kb, n, kk);   // z_t . k_i
    f32x4 w23, wn1;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * kk + r;
        const float zeta = (t >= il) ? __expf(Lv[t] - li) : 0.f;
        w23[r] = zeta * (s2[r] - s3[r]);
        wn1[r] = -zeta * s1[r];
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) BK[j] = BV[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const int t = 16 * tb + 4 * kk + s;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            BK[j] = mfma4(X[t * PD + 16 * j + n], w23[s], BK[j]);
            BK[j] = mfma4(Zt[t * PD + 16 * j + n], wn1[s], BK[j]);
            BV[j] = mfma4(Gt[t * PD + 16 * j + n], -wn1[s], BV[j]);
        }
    }
}

template <int D, int C, int W, typename In>
__device__ __forceinline__ void kv_wave(KvLds<D, C>& L, int lane, const In* __restrict__ k,
                                        const In* __restrict__ v, size_t tok0, int valid,
                                        const float* __restrict__ Pgx, const float* __restrict__ Pzx,
                                        const int* __restrict__ Egx, const int* __restrict__ Ezx,
                                        float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ akey) {
    constexpr int NT = D / 16;
    constexpr int NW = C / 16;
    constexpr int PD = lds_pitch(D);
    const int n = lane & 15, kk = lane >> 4;
    const int il = 16 * W + n;          // chunk-local key index of the lane
    const bool key_ok = il < valid;
    const float* X = L.R;
    const float* Zt = L.R + C * PD;
    const float* Gt = L.R + 2 * C * PD;

    f32x4 Kb[NT], Vb[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const size_t off = (tok0 + il) * D + 16 * j + 4 * kk;
        Kb[j] = key_ok ? load4(k + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        Vb[j] = key_ok ? load4(v + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // ---- the later chunks, through the reverse states (while the tiles land) ----
    f32x4 DV[NT], DK[NT];
    if constexpr (D >= 32) state_terms_h2<D>(Pgx, Pzx, Egx, Ezx, lane, Kb, Vb, DV, DK, L.Tr[W]);
    else state_terms<D>(Pgx, Pzx, lane, Kb, Vb, DV, DK, L.Tr[W]);
    __builtin_amdgcn_s_waitcnt(0);   // this wave's direct tile loads are in LDS
    __syncthreads();                 // and every wave's, and the log decays
    const float li = L.L[il];
    const float es = __expf(L.L[C - 1] - li);   // e^{l_end - l_i}
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            DV[j][r] *= es;
            DK[j][r] *= es;
        }

    // ---- within the chunk: tokens t >= i, one 16-token block at a time ----
    // Each block's sums are fresh MFMA chains, added into DK, DV on the VALU.
    // With four waves, wave 0 leaves its last block (token block 3) to wave 3.
    constexpr bool RB = kv_rebalance<C>();
    constexpr int TB_END = RB && W == 0 ? NW - 1 : NW;
#pragma unroll 1
    for (int tb = W; tb < TB_END; ++tb) {
        f32x4 BK[NT], BV[NT];
        kv_pair<D>(X, Zt, Gt, L.L, tb, Kb, Vb, il, li, n, kk, BK, BV);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            DK[j] += BK[j];
            DV[j] += BV[j];
        }
    }

    // ---- outputs ----
    auto outputs = [&]() {
        float vd = 0.f, kd = 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                vd += Vb[j][r] * DV[j][r];
                kd += Kb[j][r] * DK[j][r];
            }
            if (key_ok) {
                store_row(dv + (tok0 + il) * D + 16 * j + 4 * kk, DV[j]);
                store_row(dk + (tok0 + il) * D + 16 * j + 4 * kk, DK[j]);
            }
        }
        const float a = 0.5f * (kslot_sum(vd) + kslot_sum(kd));
        if (key_ok && kk == 0) akey[tok0 + il] = a;
    };
    if constexpr (!RB) {
        outputs();
    } else if constexpr (W == 0) {
        // key block 0's sums over token block 3, from wave 3
        __syncthreads();
        const float* pk = L.Pk0 + lane * 4;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            DK[j] += ld4(pk + 64 * 4 * j);
            DV[j] += ld4(pk + 64 * 4 * (NT + j));
        }
        outputs();
    } else if constexpr (W == NW - 1) {
        outputs();
        // key block 0 (keys 0..15) over token block 3, for wave 0
        f32x4 K0[NT], V0[NT];
        const bool ok0 = n < valid;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const size_t off = (tok0 + n) * D + 16 * j + 4 * kk;
            K0[j] = ok0 ? load4(k + off) : f32x4{0.f, 0.f, 0.f, 0.f};
            V0[j] = ok0 ? load4(v + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        }
        f32x4 BK[NT], BV[NT];
        kv_pair<D>(X, Zt, Gt, L.L, NW - 1, K0, V0, n, L.L[n], n, kk, BK, BV);
        float* pk = L.Pk0 + lane * 4;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            *reinterpret_cast<f32x4*>(pk + 64 * 4 * j) = BK[j];
            *reinterpret_cast<f32x4*>(pk + 64 * 4 * (NT + j)) = BV[j];
        }
        __syncthreads();
    } else {
        outputs();
        __syncthreads();
    }
}

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void bwd_kv_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma,
    const float* __restrict__ x, const float* __restrict__ z, const float* __restrict__ gout,
    const float* __restrict__ Pgx, const float* __restrict__ Pzx, const int* __restrict__ Egx,
    const int* __restrict__ Ezx, int T, int n_chunks,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ akey) {
    constexpr int NW = C / 16;
    constexpr int PD = lds_pitch(D);
    __shared__ KvLds<D, C> L;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x % n_chunks;
    const long bh = blockIdx.x / n_chunks;
    const int t0 = c * C;
    const int valid = min(C, T - t0);
    const size_t tok0 = (size_t)bh * T + t0;
    const size_t soff = ((size_t)bh * n_chunks + c) * D * D;   // P^gx, M: accumulator order

    // ---- x, z, g rows of the chunk straight into LDS (rows past the end zeroed); l ----
    // One row per wave instruction: lanes 0..D/4-1 each move 16 bytes.
    const float* srcs[3] = {x, z, gout};
    for (int e = w; e < 3 * C; e += NW) {
        const int which = e / C, r = e % C;
        float* row = L.R + which * C * PD + r * PD;
        if (lane < D / 4) {
            if (r < valid)
                __builtin_amdgcn_global_load_lds(srcs[which] + (tok0 + r) * D + 4 * lane,
                                                 (__attribute__((address_space(3))) void*)row, 16, 0, 0);
            else
                *reinterpret_cast<f32x4*>(row + 4 * lane) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    if (w == 0) {
        const float l = chunk_log_decay(gamma + tok0, valid, lane);
        if (lane < C) L.L[lane] = l;
    }

    const float* pg = Pgx + soff;
    const float* pz = Pzx + soff;
    const size_t eoff = ((size_t)bh * n_chunks + c) * (D / 16);   // the states' exponents (d >= 32)
    const int* eg = Egx + eoff;
    const int* ez = Ezx + eoff;
    if (w == 0) {
        kv_wave<D, C, 0, In>(L, lane, k, v, tok0, valid, pg, pz, eg, ez, dk, dv, akey);
    } else if constexpr (NW > 1) {
        if (w == 1) {
            kv_wave<D, C, 1, In>(L, lane, k, v, tok0, valid, pg, pz, eg, ez, dk, dv, akey);
        } else if constexpr (NW > 2) {
            if (w == 2) kv_wave<D, C, 2, In>(L, lane, k, v, tok0, valid, pg, pz, eg, ez, dk, dv, akey);
            else kv_wave<D, C, 3, In>(L, lane, k, v, tok0, valid, pg, pz, eg, ez, dk, dv, akey);
        }
    }
}

template <int D, int C, typename In>
static hipError_t launch_t(const BwdKvArgs& a, hipStream_t s) {
    const long grid = a.BH * a.n_chunks;
    hipLaunchKernelGGL((bwd_kv_kernel<D, C, In>), dim3((unsigned)grid), dim3(64 * (C / 16)), 0, s, (const In*)a.k,
                       (const In*)a.v, a.gamma, a.x, a.z, a.gout, a.Pgx, a.Pzx, a.Egx, a.Ezx, a.T, a.n_chunks, a.dk,
                       a.dv, a.akey);
    return hipGetLastError();
}

template <int D, typename In>
static hipError_t dispatch_c(const BwdKvArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_t<D, 16, In>(a, s);
        case 32: return launch_t<D, 32, In>(a, s);
        case 64: return launch_t<D, 64, In>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename In>
static hipError_t dispatch_d(const BwdKvArgs& a, hipStream_t s) {
    switch (a.d) {
        case 16: return dispatch_c<16, In>(a, s);
        case 32: return dispatch_c<32, In>(a, s);
        case 64: return dispatch_c<64, In>(a, s);
        case 128: return dispatch_c<128, In>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_kv(const BwdKvArgs& a, hipStream_t s) {
    return a.bf16 ? dispatch_d<bf16_t>(a, s) : dispatch_d<float>(a, s);
}

}  // namespace mesa
