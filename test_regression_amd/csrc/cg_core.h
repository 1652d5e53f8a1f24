// cg_core.h -- the chunk-local CG machinery shared by the forward CG kernel
// and the backward's adjoint solve (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section "A Camada
// Mesa": the output is Delta_t = G_t q*_t with q*_t = (H_t + Lambda)^{-1}
// q_t solved by Conjugate Gradient; bullet "Paralelizacao": CG over all time
// steps is a gated-linear-attention pass run chunk-parallel on the states.
// For chunk c (tokens t0..t0+C-1, l_t the within-chunk prefix sum of
// ln gamma, S^H_c = H_{t0-1}):
//   H_t p = e^{l_t} S^H_c p + sum_{i=t0..t} e^{l_t - l_i} (k_i . p) k_i
//
// Layout (see the kernels for the full story): one workgroup per (head,
// chunk), wave w owns tokens 16w..16w+15; every product is computed
// transposed so that a wave's vectors (lane (n, kk) holds features
// 16j + 4kk + r of token n in block j) are the MFMA B operand and the LDS
// tiles are the A operand.  Every MFMA chain starts from zero and is only
// read afterwards.
#pragma once
#include "mesa_device.h"

namespace mesa {


constexpr int kBlockPitch = 20;   // floats per row of a stored 16x16 state block

template <int D, int C>
struct alignas(16) CgLds {
    static constexpr int NW = C / 16;
    static constexpr int NT = D / 16;
    static constexpr int NBLK = NT * (NT + 1) / 2;       // upper-triangle blocks
    static constexpr int HALF = NBLK * 16 * kBlockPitch;  // floats per stored state
    static constexpr int NSTATE = NW >= 2 ? 2 : 1;
    static constexpr int PD = lds_pitch(D);
    static constexpr int PS = lds_pitch_rows(D);
    static constexpr int PT = lds_pitch_rows(C);
    float R[NSTATE * HALF];   // stored S^H_c [, S_mid]
    float KV[C * PD];         // K_c rows [token][feature]
    float KT[D * PT];         // K_c^T, later V_c^T   [feature][token]
    float L[C];               // l_i
    float Lam[D];
    int next;                 // the forward kernel's claimed next chunk
};

__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// An LDS float pointer held as a 32-bit LDS address.
typedef const __attribute__((address_space(3))) float lds_cfloat;

// Index of stored block (a, b), a <= b, in the packed NT x NT upper block triangle.
template <int NT>
__host__ __device__ constexpr int blk_index(int a, int b) { return a * NT - a * (a - 1) / 2 + (b - a); }

// Offset (floats) of stored block (a, b), a <= b, of an NT x NT block triangle.
template <int NT>
__host__ __device__ constexpr int blk(int a, int b) {
    return (a * NT - a * (a - 1) / 2 + (b - a)) * 16 * kBlockPitch;
}

// Y[j]   += S[16j + m][:] . Z^T[:][n]                 (S symmetric, upper block triangle stored)
// Sc[ib] += K[16(KB0 + ib) + m][:] . Z^T[:][n]        (NB score blocks)
// Z: the wave's vectors in registers (lane (n, kk), block g: features 16g + 4kk + s of token n).
// S[16j + m][16g + 4kk + s] is stored block (j, g) read along row m when j < g,
// else block (g, j) read down column m (S symmetric).
// col[blk_index(g, j)]: the lane's column-read address in stored block (g, j).
template <int D, int NB, int KB0>
__device__ __forceinline__ void contract_state_scores(const f32x4 (&Z)[D / 16], const float* Sst,
                                                      lds_cfloat* const (&col)[D / 16 * (D / 16 + 1) / 2],
                                                      const float* Kr, int m, int kk, f32x4 (&Y)[D / 16],
                                                      f32x4 (&Sc)[NB]) {
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    f32x4 bs[2][NT], bk[2][NB];
    auto load = [&](int g, int buf) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (g > j) {
                bs[buf][j] = lds4(Sst + blk<NT>(j, g) + m * kBlockPitch + 4 * kk);
            } else {
                lds_cfloat* c = col[blk_index<NT>(g, j)];
#pragma unroll
                for (int s = 0; s < 4; ++s) bs[buf][j][s] = c[s * kBlockPitch];
            }
        }
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) bk[buf][ib] = lds4(Kr + (16 * (KB0 + ib) + m) * PD + 16 * g + 4 * kk);
    };
    load(0, 0);
#pragma unroll
    for (int g = 0; g < NT; ++g) {
        const int cur = g & 1;
        if (g + 1 < NT) load(g + 1, cur ^ 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int j = 0; j < NT; ++j) Y[j] = mfma4(bs[cur][j][s], Z[g][s], Y[j]);
#pragma unroll
            for (int ib = 0; ib < NB; ++ib) Sc[ib] = mfma4(bk[cur][ib][s], Z[g][s], Sc[ib]);
        }
    }
}

// Y[j] += Bs[16j + m][:] . Z^T[:][n]  (Bs full, row-major, pitch lds_pitch_rows(D)), when STATE;
// Sc[ib] += K[16ib + m][:] . Z^T[:][n] for ib < NB (K rows, pitch lds_pitch(D)).
template <int D, int NB, bool STATE>
__device__ __forceinline__ void contract_rows(const f32x4 (&Z)[D / 16], const float* Bs, const float* Bk, int m,
                                              int kk, f32x4 (&Y)[D / 16], f32x4 (&Sc)[NB > 0 ? NB : 1]) {
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    constexpr int PS = lds_pitch_rows(D);
    constexpr int NBB = NB > 0 ? NB : 1;
    const float* bsa = STATE ? Bs + m * PS + 4 * kk : nullptr;
    const float* bka = NB > 0 ? Bk + m * PD + 4 * kk : nullptr;
    f32x4 bs[2][STATE ? NT : 1], bk[2][NBB];
    auto load = [&](int g, int buf) {
        if constexpr (STATE) {
#pragma unroll
            for (int j = 0; j < NT; ++j) bs[buf][j] = lds4(bsa + 16 * j * PS + 16 * g);
        }
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) bk[buf][ib] = lds4(bka + 16 * ib * PD + 16 * g);
    };
    load(0, 0);
#pragma unroll
    for (int g = 0; g < NT; ++g) {
        const int cur = g & 1;
        if (g + 1 < NT) load(g + 1, cur ^ 1);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if constexpr (STATE) {
#pragma unroll
                for (int j = 0; j < NT; ++j) Y[j] = mfma4(bs[cur][j][s], Z[g][s], Y[j]);
            }
#pragma unroll
            for (int ib = 0; ib < NB; ++ib) Sc[ib] = mfma4(bk[cur][ib][s], Z[g][s], Sc[ib]);
        }
    }
}

// Y[j] += sum_{ib < NB} sum_i BT[16j + m][16(KB0 + ib) + i] * W[ib][i]
// BT: K^T or V^T tile [feature][token] (pitch lds_pitch_rows(C));
// W: decayed score blocks in registers (lane (n, kk): keys 16(KB0 + ib) + 4kk + s of token n).
template <int D, int C, int NB, int KB0>
__device__ __forceinline__ void contract_intra(const f32x4 (&W)[NB], const float* BT, int m, int kk,
                                               f32x4 (&Y)[D / 16]) {
    constexpr int NT = D / 16;
    constexpr int PT = lds_pitch_rows(C);
    const float* base = BT + m * PT + 16 * KB0 + 4 * kk;
    f32x4 a[2][NT];
    auto load = [&](int ib, int buf) {
#pragma unroll
        for (int j = 0; j < NT; ++j) a[buf][j] = lds4(base + 16 * j * PT + 16 * ib);
    };
    load(0, 0);
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
        const int cur = ib & 1;
        if (ib + 1 < NB) load(ib + 1, cur ^ 1);
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int j = 0; j < NT; ++j) Y[j] = mfma4(a[cur][j][s], W[ib][s], Y[j]);
    }
}

// S_mid (upper block triangle) = e^{l_{h-1}} S0 + sum_{i<h} e^{l_{h-1}-l_i} k_i k_i^T,
// blocks distributed over the NW waves.  Written to S1.
template <int D, int C>
__device__ __forceinline__ void form_mid_state(CgLds<D, C>& L, int w, int n, int kk) {
    constexpr int NT = D / 16;
    constexpr int NW = C / 16;
    constexpr int H = C / 2;
    constexpr int PD = lds_pitch(D);
    const float* S0 = L.R;
    float* S1 = L.R + CgLds<D, C>::HALF;
    const float lh = L.L[H - 1];
    const float Gh = __expf(lh);
    // Token of k-slot group kk in step st: (st mod 4) + 4kk + 16(st / 4).  Its
    // K row then starts at bank 4(st mod 4) + 16kk (the row pitch is 4 mod
    // 64 banks), so the 64 lanes' reads hit distinct banks.
    auto tok = [&](int st) { return (st & 3) + 4 * kk + 16 * (st >> 2); };
    float wk[H / 4];
#pragma unroll
    for (int st = 0; st < H / 4; ++st) wk[st] = __expf(lh - L.L[tok(st)]);
    int q = 0;
#pragma unroll
    for (int a = 0; a < NT; ++a) {
#pragma unroll
        for (int b = a; b < NT; ++b, ++q) {
            if (q % NW != w) continue;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < H / 4; ++st) {
                const int i = tok(st);
                acc = mfma4(wk[st] * L.KV[i * PD + 16 * a + n], L.KV[i * PD + 16 * b + n], acc);
            }
            const float* s0 = S0 + blk<NT>(a, b) + (4 * kk) * kBlockPitch + n;
            float* s1 = S1 + blk<NT>(a, b) + (4 * kk) * kBlockPitch + n;
#pragma unroll
            for (int r = 0; r < 4; ++r) s1[r * kBlockPitch] = Gh * s0[r * kBlockPitch] + acc[r];
        }
    }
}


// Per-wave constants of wave W in chunk-local CG work.
template <int D, int C, int W>
struct CgWave {
    static constexpr int NT = D / 16;
    static constexpr int NW = C / 16;
    static constexpr int SUB = (NW >= 2 && W >= NW / 2) ? 1 : 0;   // which stored state
    static constexpr int KB0 = SUB ? NW / 2 : 0;                    // first key block of the sub-chunk
    static constexpr int NB = W - KB0 + 1;                          // causal key blocks in the CG
    static constexpr int NBO = W + 1;                               // causal key blocks over the chunk
    int n, kk, tr;        // lane's token (B column), k-slot group, chunk token
    float eL, eLo;        // e^{l_t - l_base} (sub-chunk state), e^{l_t} (chunk-start state)
    static constexpr int NCOL = NT * (NT + 1) / 2;
    float dec[NBO][4];    // e^{l_t - l_i} for key i = 16ib + 4kk + r <= t, else 0
    const float* Sst;     // the stored state the CG uses
    // Column-read addresses (row 4kk, column n) of the stored blocks.  Each
    // is passed through an empty asm so that the compiler keeps it in a
    // register across the CG loop rather than rebuilding it there from a
    // base and a constant (the 8-bit offsets of two-address LDS reads reach
    // only 1 KiB).
    lds_cfloat* col[NCOL];

    __device__ __forceinline__ CgWave(const CgLds<D, C>& L, int lane) {
        n = lane & 15;
        kk = lane >> 4;
        tr = 16 * W + n;
        Sst = L.R + SUB * CgLds<D, C>::HALF;
#pragma unroll
        for (int a = 0; a < NT; ++a)
#pragma unroll
            for (int b = a; b < NT; ++b) {
                lds_cfloat* c = (lds_cfloat*)(Sst + blk<NT>(a, b) + (4 * kk) * kBlockPitch + n);
                asm volatile("" : "+v"(c));
                col[blk_index<NT>(a, b)] = c;
            }
        const float lbase = SUB ? L.L[16 * KB0 - 1] : 0.f;   // l at the end of the first half
        eL = __expf(L.L[tr] - lbase);
        eLo = __expf(L.L[tr]);
#pragma unroll
        for (int ib = 0; ib < NBO; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int i = 16 * ib + 4 * kk + r;
                dec[ib][r] = (i <= tr) ? __expf(L.L[tr] - L.L[i]) : 0.f;
            }
    }
};

// Dot product of each token's vectors held in B layout (the four k-slot lanes
// of a token end with the same bits).
template <int NT>
__device__ __forceinline__ float token_dot(const f32x4 (&A)[NT], const f32x4 (&B)[NT]) {
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[r] += A[j][r] * B[j][r];
    return kslot_sum((s[0] + s[1]) + (s[2] + s[3]));
}

// num / den through the hardware reciprocal (about 1 ulp).  The reciprocal
// flushes a denormal input to zero, so a denominator below the smallest normal
// float is scaled by 2^64 first and the quotient scaled back: a token that
// keeps iterating after its residual has shrunk to denormal size (fixed
// iteration counts far past convergence) keeps finite alpha and beta.
__device__ __forceinline__ float rcp_div(float num, float den) {
    const float s = den < 1.17549435e-38f ? 0x1p64f : 1.0f;
    return (num * __builtin_amdgcn_rcpf(den * s)) * s;
}

// Y = H_t P over the wave's tokens (the stored state plus the sub-chunk's
// causal keys), plus diag(lambda) P when LAMBDA: one CG matvec.
template <int D, int C, int W, bool LAMBDA>
__device__ __forceinline__ void wave_matvec(const CgLds<D, C>& L, const CgWave<D, C, W>& cw,
                                            const f32x4 (&P)[D / 16], f32x4 (&Y)[D / 16]) {
    using CW = CgWave<D, C, W>;
    constexpr int NT = D / 16;
    f32x4 YS[NT], YI[NT], Sc[CW::NB];
#pragma unroll
    for (int j = 0; j < NT; ++j) YS[j] = YI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ib = 0; ib < CW::NB; ++ib) Sc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
    contract_state_scores<D, CW::NB, CW::KB0>(P, cw.Sst, cw.col, L.KV, cw.n, cw.kk, YS, Sc);
    f32x4 Wt[CW::NB];
#pragma unroll
    for (int ib = 0; ib < CW::NB; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) Wt[ib][r] = Sc[ib][r] * cw.dec[CW::KB0 + ib][r];
    contract_intra<D, C, CW::NB, CW::KB0>(Wt, L.KT, cw.n, cw.kk, YI);
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        if constexpr (LAMBDA) {
            const f32x4 lam = lds4(&L.Lam[16 * j + 4 * cw.kk]);
#pragma unroll
            for (int r = 0; r < 4; ++r) Y[j][r] = cw.eL * YS[j][r] + YI[j][r] + lam[r] * P[j][r];
        } else {
#pragma unroll
            for (int r = 0; r < 4; ++r) Y[j][r] = cw.eL * YS[j][r] + YI[j][r];
        }
    }
}

// CG on (H_t + Lambda) x = b for the wave's 16 tokens from x = 0.  R holds b
// on entry (B layout); X receives the solution.  Stops before an update when
// |r| / |b| < tol (tested as r.r < (tol |b|)^2), or on r.r == 0 or
// p.Ap <= 0; b == 0 gives x = 0 and no update.  Returns the lane's token's
// update count.  matvec(P, Y) sets Y = (H_t + Lambda) P for the wave.
template <int NT, typename Matvec>
__device__ __forceinline__ int cg_solve(f32x4 (&R)[NT], f32x4 (&X)[NT], int max_iters, float tol,
                                        const Matvec& matvec) {
    f32x4 P[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        P[j] = R[j];
        X[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float rr = token_dot<NT>(R, R);
    const float tq = tol * sqrtf(rr);
    const float stop_rr = tq * tq;
    bool done = !(rr > 0.f);   // b == 0 (or a padded token): x = 0, 0 iterations
    int it = 0;
    for (int itn = 0; itn < max_iters; ++itn) {
        if (!done && (rr < stop_rr || rr == 0.f)) done = true;
        if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
        f32x4 Y[NT];
        matvec(P, Y);
        const float pap = token_dot<NT>(P, Y);
        const bool act = !done && (pap > 0.f);
        if (!done && !act) done = true;   // breakdown guard
        // alpha and beta divide through the hardware reciprocal (about 1 ulp
        // instead of a correctly rounded division sequence), see rcp_div.
        const float alpha = act ? rcp_div(rr, pap) : 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                X[j][r] += alpha * P[j][r];
                R[j][r] -= alpha * Y[j][r];
            }
        const float rrn = token_dot<NT>(R, R);
        // Written for every lane (a stopped token gets beta = 0, so its
        // direction becomes its frozen residual and stays finite): a lane-
        // conditional update made the compiler copy P between register
        // ranges at the end of every iteration.
        const float beta = act ? rcp_div(rrn, rr) : 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) P[j][r] = R[j][r] + beta * P[j][r];
        rr = act ? rrn : rr;
        it += act ? 1 : 0;
    }
    return it;
}

// cg_solve with the matvec in two parts: head(P) reads only P's first two
// 16-feature blocks, rest(P, Y) completes Y = (H_t + Lambda) P.  Each
// iteration updates those two blocks of P first and issues the next head
// before the other blocks' x and p updates, so the next matvec's first
// MFMAs overlap them.  The arithmetic is cg_solve's, element for element;
// after the last iteration the head's work is discarded.
template <int NT, typename Head, typename Rest>
__device__ __forceinline__ int cg_solve_pipelined(f32x4 (&R)[NT], f32x4 (&X)[NT], int max_iters, float tol,
                                                  const Head& head, const Rest& rest) {
    f32x4 P[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        P[j] = R[j];
        X[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float rr = token_dot<NT>(R, R);
    const float tq = tol * sqrtf(rr);
    const float stop_rr = tq * tq;
    bool done = !(rr > 0.f);   // b == 0 (or a padded token): x = 0, 0 iterations
    int it = 0;
    if (max_iters > 0) head(P);
    for (int itn = 0; itn < max_iters; ++itn) {
        if (!done && (rr < stop_rr || rr == 0.f)) done = true;
        if (__builtin_amdgcn_ballot_w64(!done) == 0) break;
        f32x4 Y[NT];
        rest(P, Y);
        const float pap = token_dot<NT>(P, Y);
        const bool act = !done && (pap > 0.f);
        if (!done && !act) done = true;   // breakdown guard
        const float alpha = act ? rcp_div(rr, pap) : 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) R[j][r] -= alpha * Y[j][r];
        const float rrn = token_dot<NT>(R, R);
        const float beta = act ? rcp_div(rrn, rr) : 0.f;
        constexpr int J0 = NT >= 2 ? 2 : NT;
#pragma unroll
        for (int j = 0; j < J0; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                X[j][r] += alpha * P[j][r];
                P[j][r] = R[j][r] + beta * P[j][r];
            }
        head(P);
#pragma unroll
        for (int j = J0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                X[j][r] += alpha * P[j][r];
                P[j][r] = R[j][r] + beta * P[j][r];
            }
        rr = act ? rrn : rr;
        it += act ? 1 : 0;
    }
    return it;
}

// The chunk-local CG of wave W: Y = (H_t + Lambda) P from the LDS tiles.
template <int D, int C, int W>
__device__ __forceinline__ int cg_solve_wave(const CgLds<D, C>& L, const CgWave<D, C, W>& cw, f32x4 (&R)[D / 16],
                                             f32x4 (&X)[D / 16], int max_iters, float tol) {
    return cg_solve<D / 16>(R, X, max_iters, tol, [&](const f32x4 (&P)[D / 16], f32x4 (&Y)[D / 16]) {
        wave_matvec<D, C, W, true>(L, cw, P, Y);
    });
}

// Stage the stored upper block triangle of S^H (blocks (a, b), a <= b, in
// row-major block order, each block in accumulator order) into L.R as
// row-major blocks of pitch kBlockPitch; workgroup-wide.
template <int D, int C>
__device__ __forceinline__ void stage_packed_state(CgLds<D, C>& L, const float* __restrict__ SHc, int tid,
                                                   int nthr) {
    constexpr int HPACK = D * (D + 16) / 2;
    for (int e = tid * 4; e < HPACK; e += nthr * 4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(SHc + e);   // rows 4kk..4kk+3 of column n
        const int l = (e % 256) / 4, kk = l / 16, n = l % 16;
        float* dst = &L.R[(e / 256) * 16 * kBlockPitch + (4 * kk) * kBlockPitch + n];
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[r * kBlockPitch] = v[r];
    }
}

// The stored upper block triangle of S^H (as stage_packed_state reads it)
// held in registers between its global load and its LDS store.
template <int D, int NTHR>
struct PackedStateRegs {
    static constexpr int HPACK = D * (D + 16) / 2;
    static constexpr int N = (HPACK + 4 * NTHR - 1) / (4 * NTHR);
    f32x4 x[N];
    __device__ __forceinline__ void load(const float* __restrict__ src, int tid) {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int e = (tid + u * NTHR) * 4;
            if (e < HPACK) x[u] = *reinterpret_cast<const f32x4*>(src + e);
        }
    }
    __device__ __forceinline__ void store(float* R, int tid) const {
#pragma unroll
        for (int u = 0; u < N; ++u) {
            const int e = (tid + u * NTHR) * 4;
            if (e < HPACK) {
                const int l = (e % 256) / 4, kk = l / 16, n = l % 16;
                float* dst = R + (e / 256) * 16 * kBlockPitch + (4 * kk) * kBlockPitch + n;
#pragma unroll
                for (int r = 0; r < 4; ++r) dst[r * kBlockPitch] = x[u][r];
            }
        }
    }
};

// A chunk's rows of a [*, D] tensor held in registers between their global
// load and their transposed store to LDS (pitch lds_pitch_rows(C)), so the
// loads can be issued before the LDS tile is free; rows past `valid` are zero.
template <int D, int C, int NTHR, typename In>
struct ChunkRowsRegs {
    static constexpr int EL4 = C * D / (4 * NTHR);
    static_assert(C * D % (4 * NTHR) == 0, "tile must split evenly over the workgroup");
    Raw4<In> x[EL4];   // bf16 stays packed until stored
    // Group u of a thread: token i, features f..f+3.  Four neighbouring lanes
    // take 16 consecutive features of one token and a wave 16 tokens, so the
    // transposed stores of a wave hit distinct LDS banks but for a 2-way
    // overlap (one token per lane group would put 16 lanes on a bank).
    __device__ __forceinline__ static void place(int u, int tid, int& i, int& f) {
        const int e4 = tid + u * NTHR;
        i = (e4 >> 2) % C;
        f = 16 * (e4 / (4 * C)) + 4 * (e4 & 3);
    }
    __device__ __forceinline__ void load(const In* __restrict__ src, int valid, int tid) {
#pragma unroll
        for (int u = 0; u < EL4; ++u) {
            int i, f;
            place(u, tid, i, f);
            x[u].zero();
            if (i < valid) x[u].load(src + (size_t)i * D + f);
        }
    }
    __device__ __forceinline__ void store_rows(float* rows, int tid) const {
        constexpr int PD = lds_pitch(D);
#pragma unroll
        for (int u = 0; u < EL4; ++u) {
            int i, f;
            place(u, tid, i, f);
            *reinterpret_cast<f32x4*>(&rows[i * PD + f]) = x[u].get();
        }
    }
    __device__ __forceinline__ void store_transposed(float* tr, int tid) const {
        constexpr int PT = lds_pitch_rows(C);
#pragma unroll
        for (int u = 0; u < EL4; ++u) {
            int i, f;
            place(u, tid, i, f);
#pragma unroll
            for (int r = 0; r < 4; ++r) tr[(f + r) * PT + i] = x[u].get()[r];
        }
    }
};

}  // namespace mesa
