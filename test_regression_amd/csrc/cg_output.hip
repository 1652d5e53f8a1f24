// cg_output.hip -- all CG iterations of one chunk plus the output contraction
// of the Mesa layer (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section "A Camada
// Mesa":
//  - the output is Delta_t = G_t q*_t with q*_t = (H_t + Lambda)^{-1} q_t,
//    solved by Conjugate Gradient (sentence after the displayed objective);
//  - bullet "Paralelizacao": CG over all time steps is a gated-linear-
//    attention pass and runs chunk-parallel on the states H_t, G_t;
//  - bullet "Computacao Dinamica": the iteration count varies per token.
//
// Chunkwise form (chunk c covers tokens t0..t0+C-1, l_t the within-chunk
// prefix sum of ln gamma, S^H_c = H_{t0-1}, S^G_c = G_{t0-1}):
//   H_t p = e^{l_t} S^H_c p + sum_{i=t0..t} e^{l_t - l_i} (k_i . p) k_i
//   G_t x = e^{l_t} S^G_c x + sum_{i=t0..t} e^{l_t - l_i} (k_i . x) v_i
// The keys are both the "keys" and the "values" of the CG matvec and never
// change between iterations, so everything the matvec needs stays in LDS.
//
// Sub-chunk states.  H is symmetric, so only the upper triangle of 16x16
// blocks of a state is kept in LDS; that leaves room for a second state,
//   S_mid = H_{t0+h-1} = e^{l_{h-1}} S^H_c + sum_{i<h} e^{l_{h-1}-l_i} k_i k_i^T,
// the state at the middle of the chunk (h = C/2), formed once per chunk.
// Tokens in the second half then use S_mid and need intra-chunk terms only
// against the keys of the second half.
//
// Work split: one workgroup per (head, chunk); wave w owns tokens
// 16w..16w+15 and runs their CG entirely on its own: the tiles in LDS are
// read-only during the iterations, so the CG loop has no workgroup barrier
// and waves stop independently.  Each wave runs a body specialised on w
// (static sub-chunk, causal block range).
//
// Transposed products.  Every contraction is computed as its transpose,
// e.g. Y^T = S P^T with the state as the MFMA A operand and the wave's CG
// vectors as the B operand (v_mfma_f32_16x16x4_f32).  In that form the B
// operand a lane supplies (token n, four consecutive features) is exactly
// what it holds of the result: lane (n, kk) keeps features 16j + 4kk + r of
// token n in block j.  So the CG vectors and the decayed scores feed the next
// MFMA straight from registers, the loop writes nothing to LDS, and each
// token's alpha/beta dot products finish with two lane swaps over its four
// k-slot lanes.  The A operands (state rows, key rows, K^T rows) are 128-bit
// LDS reads, issued one k-group ahead of the MFMAs that use them.  Every MFMA
// chain starts from zero and is only read afterwards.
#include "mesa_device.h"
#include "mesa_kernels.h"

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
    static constexpr int REGION = NSTATE * HALF > D * PS ? NSTATE * HALF : D * PS;
    float R[REGION];          // CG: stored S^H_c [, S_mid];  output: G_c full [D][PS]
    float KV[C * PD];         // K_c rows [token][feature]
    float KT[D * PT];         // K_c^T, later V_c^T   [feature][token]
    float L[C];               // l_i
    float Lam[D];
};

__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

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
template <int D, int NB, int KB0>
__device__ __forceinline__ void contract_state_scores(const f32x4 (&Z)[D / 16], const float* Sst, const float* Kr,
                                                      int m, int kk, f32x4 (&Y)[D / 16], f32x4 (&Sc)[NB]) {
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    f32x4 bs[2][NT], bk[2][NB];
    auto load = [&](int g, int buf) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (g > j) {
                bs[buf][j] = lds4(Sst + blk<NT>(j, g) + m * kBlockPitch + 4 * kk);
            } else {
                const float* col = Sst + blk<NT>(g, j) + (4 * kk) * kBlockPitch + m;
#pragma unroll
                for (int s = 0; s < 4; ++s) bs[buf][j][s] = col[s * kBlockPitch];
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
    float wk[H / 4];
#pragma unroll
    for (int st = 0; st < H / 4; ++st) wk[st] = __expf(lh - L.L[4 * st + kk]);
    int q = 0;
#pragma unroll
    for (int a = 0; a < NT; ++a) {
#pragma unroll
        for (int b = a; b < NT; ++b, ++q) {
            if (q % NW != w) continue;
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < H / 4; ++st) {
                const int i = 4 * st + kk;
                acc = mfma4(wk[st] * L.KV[i * PD + 16 * a + n], L.KV[i * PD + 16 * b + n], acc);
            }
            const float* s0 = S0 + blk<NT>(a, b) + (4 * kk) * kBlockPitch + n;
            float* s1 = S1 + blk<NT>(a, b) + (4 * kk) * kBlockPitch + n;
#pragma unroll
            for (int r = 0; r < 4; ++r) s1[r * kBlockPitch] = Gh * s0[r * kBlockPitch] + acc[r];
        }
    }
}

// The CG of wave W (tokens 16W..16W+15 of the chunk) and its output rows.
template <int D, int C, int W, typename In>
__device__ __forceinline__ void cg_wave(CgLds<D, C>& L, int tid, const In* __restrict__ q,
                                        const In* __restrict__ v, const float* __restrict__ Gc, size_t tok0,
                                        int valid, int max_iters, float tol, float* __restrict__ out,
                                        int32_t* __restrict__ iters) {
    constexpr int NT = D / 16;
    constexpr int NW = C / 16;
    constexpr int SUB = (NW >= 2 && W >= NW / 2) ? 1 : 0;   // which stored state
    constexpr int KB0 = SUB ? NW / 2 : 0;                    // first key block of the sub-chunk
    constexpr int NB = W - KB0 + 1;                          // causal key blocks in the CG
    constexpr int NBO = W + 1;                               // causal key blocks of the output
    constexpr int PS = lds_pitch_rows(D);
    constexpr int PT = lds_pitch_rows(C);
    constexpr int NTHR = 64 * NW;
    const int lane = tid & 63;
    const int n = lane & 15;    // token of the lane (B operand / result column)
    const int kk = lane >> 4;   // k-slot group (features 4kk..4kk+3 of each block)
    const float* Sst = L.R + SUB * CgLds<D, C>::HALF;
    const int tr = 16 * W + n;  // chunk token of this lane
    const bool tok_ok = tr < valid;

    // ---- per-lane constants ----
    const float lbase = SUB ? L.L[16 * KB0 - 1] : 0.f;   // l at the end of the first half
    const float eL = __expf(L.L[tr] - lbase);
    const float eLo = __expf(L.L[tr]);
    float dec[NBO][4];   // e^{l_t - l_i} for key i = 16ib + 4kk + r <= t, else 0
#pragma unroll
    for (int ib = 0; ib < NBO; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int i = 16 * ib + 4 * kk + r;
            dec[ib][r] = (i <= tr) ? __expf(L.L[tr] - L.L[i]) : 0.f;
        }

    // ---- CG state: x = 0, r = p = q ----
    f32x4 X[NT], R[NT], P[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        R[j] = tok_ok ? load4(q + (tok0 + tr) * D + 16 * j + 4 * kk) : f32x4{0.f, 0.f, 0.f, 0.f};
        P[j] = R[j];
        X[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    auto dot = [&](const f32x4 (&A)[NT], const f32x4 (&B)[NT]) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) s += A[j][r] * B[j][r];
        return kslot_sum(s);
    };
    // stop before an update when |r| / |q| < tol, tested as r.r < (tol |q|)^2
    float rr = dot(R, R);
    const float tq = tol * sqrtf(rr);
    const float stop_rr = tq * tq;
    bool done = !(rr > 0.f);   // q_t == 0 (or a padded token): x = 0, 0 iterations
    int it = 0;

    // ---- CG iterations ----
    for (int itn = 0; itn < max_iters; ++itn) {
        if (!done && (rr < stop_rr || rr == 0.f)) done = true;
        if (__builtin_amdgcn_ballot_w64(!done) == 0) break;

        // Y = diag(e^{l - lbase}) P S + (M o (P K^T)) K + P diag(lambda) over
        // the sub-chunk, transposed; state and intra-chunk sums in separate chains.
        f32x4 Y[NT];
        {
            f32x4 YS[NT], YI[NT], Sc[NB];
#pragma unroll
            for (int j = 0; j < NT; ++j) YS[j] = YI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ib = 0; ib < NB; ++ib) Sc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
            contract_state_scores<D, NB, KB0>(P, Sst, L.KV, n, kk, YS, Sc);
            f32x4 Wt[NB];
#pragma unroll
            for (int ib = 0; ib < NB; ++ib)
#pragma unroll
                for (int r = 0; r < 4; ++r) Wt[ib][r] = Sc[ib][r] * dec[KB0 + ib][r];
            contract_intra<D, C, NB, KB0>(Wt, L.KT, n, kk, YI);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const f32x4 lam = lds4(&L.Lam[16 * j + 4 * kk]);
#pragma unroll
                for (int r = 0; r < 4; ++r) Y[j][r] = eL * YS[j][r] + YI[j][r] + lam[r] * P[j][r];
            }
        }

        const float pap = dot(P, Y);
        const bool act = !done && (pap > 0.f);
        if (!done && !act) done = true;   // breakdown guard
        const float alpha = act ? rr / pap : 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                X[j][r] += alpha * P[j][r];
                R[j][r] -= alpha * Y[j][r];
            }
        const float rrn = dot(R, R);
        if (act) {
            const float beta = rrn / rr;
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) P[j][r] = R[j][r] + beta * P[j][r];
            rr = rrn;
            it += 1;
        }
    }

    // ---- iteration counts ----
    if (iters && kk == 0 && tok_ok) iters[tok0 + tr] = it;

    // ---- output O = diag(e^l) X G_c^T + (M o (X K^T)) V over the whole chunk, transposed ----
    f32x4 Wo[NBO];
    {
        f32x4 Sc[NBO], unused[NT];
#pragma unroll
        for (int ib = 0; ib < NBO; ++ib) Sc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        contract_rows<D, NBO, false>(X, nullptr, L.KV, n, kk, unused, Sc);
#pragma unroll
        for (int ib = 0; ib < NBO; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) Wo[ib][r] = Sc[ib][r] * dec[ib][r];
    }
    __syncthreads();   // every wave is done with the states, K_c and K_c^T
    for (int e = tid * 4; e < D * D; e += NTHR * 4)
        *reinterpret_cast<f32x4*>(&L.R[(e / D) * PS + e % D]) = *reinterpret_cast<const f32x4*>(Gc + e);
    for (int e = tid * 4; e < C * D; e += NTHR * 4) {
        const int i = e / D, f = e % D;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i < valid) x = load4(v + (tok0 + i) * D + f);
#pragma unroll
        for (int u = 0; u < 4; ++u) L.KT[(f + u) * PT + i] = x[u];
    }
    __syncthreads();
    f32x4 OS[NT], OI[NT], none[1];
#pragma unroll
    for (int j = 0; j < NT; ++j) OS[j] = OI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    contract_rows<D, 0, true>(X, L.R, nullptr, n, kk, OS, none);
    contract_intra<D, C, NBO, 0>(Wo, L.KT, n, kk, OI);
    if (tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = eLo * OS[j][r] + OI[j][r];
            *reinterpret_cast<f32x4*>(out + (tok0 + tr) * D + 16 * j + 4 * kk) = o;
        }
    }
}

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void cg_output_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ gamma, const float* __restrict__ lambda,
    const float* __restrict__ SH, const float* __restrict__ SG, int H, int T, int n_chunks,
    int max_iters, float tol, float* __restrict__ out, int32_t* __restrict__ iters) {
    constexpr int NW = C / 16;
    constexpr int PD = lds_pitch(D);
    constexpr int PT = lds_pitch_rows(C);
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
    const size_t tok0 = (size_t)bh * T + t0;   // first token of the chunk
    constexpr int HPACK = D * (D + 16) / 2;    // packed upper block triangle of S^H
    const size_t hoff = ((size_t)bh * n_chunks + c) * HPACK;
    const size_t soff = ((size_t)bh * n_chunks + c) * D * D;

    // ---- stage S^H_c (packed 16x16 upper blocks, in blk order), K_c, K_c^T, lambda, l ----
    for (int e = tid * 4; e < HPACK; e += NTHR * 4)
        *reinterpret_cast<f32x4*>(&L.R[(e / 256) * 16 * kBlockPitch + ((e % 256) / 16) * kBlockPitch + e % 16]) =
            *reinterpret_cast<const f32x4*>(SH + hoff + e);
    for (int e = tid * 4; e < C * D; e += NTHR * 4) {
        const int i = e / D, f = e % D;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i < valid) x = load4(k + (tok0 + i) * D + f);
        *reinterpret_cast<f32x4*>(&L.KV[i * PD + f]) = x;
#pragma unroll
        for (int u = 0; u < 4; ++u) L.KT[(f + u) * PT + i] = x[u];
    }
    for (int e = tid; e < D; e += NTHR) L.Lam[e] = lambda[(size_t)h * D + e];
    if (w == 0) {
        const float l = chunk_log_decay(gamma + tok0, valid, lane);
        if (lane < C) L.L[lane] = l;
    }
    __syncthreads();
    if constexpr (NW >= 2) {
        form_mid_state<D, C>(L, w, lane & 15, lane >> 4);
        __syncthreads();
    }

    const float* Gc = SG + soff;
    if (w == 0) {
        cg_wave<D, C, 0, In>(L, tid, q, v, Gc, tok0, valid, max_iters, tol, out, iters);
    } else if constexpr (NW > 1) {
        if (w == 1) {
            cg_wave<D, C, 1, In>(L, tid, q, v, Gc, tok0, valid, max_iters, tol, out, iters);
        } else if constexpr (NW > 2) {
            if (w == 2) cg_wave<D, C, 2, In>(L, tid, q, v, Gc, tok0, valid, max_iters, tol, out, iters);
            else cg_wave<D, C, 3, In>(L, tid, q, v, Gc, tok0, valid, max_iters, tol, out, iters);
        }
    }
}

template <int D, int C, typename In>
static hipError_t launch_t(const CgOutputArgs& a, hipStream_t s) {
    const long grid = a.BH * a.n_chunks;
    hipLaunchKernelGGL((cg_output_kernel<D, C, In>), dim3((unsigned)grid), dim3(64 * (C / 16)), 0, s,
                       (const In*)a.q, (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.SH, a.SG,
                       a.H, a.T, a.n_chunks, a.max_iters, a.tol, a.out, a.iters);
    return hipGetLastError();
}

template <int D, typename In>
static hipError_t dispatch_c(const CgOutputArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_t<D, 16, In>(a, s);
        case 32: return launch_t<D, 32, In>(a, s);
        case 64: return launch_t<D, 64, In>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename In>
static hipError_t dispatch_d(const CgOutputArgs& a, hipStream_t s) {
    switch (a.d) {
        case 16: return dispatch_c<16, In>(a, s);
        case 32: return dispatch_c<32, In>(a, s);
        case 64: return dispatch_c<64, In>(a, s);
        case 128: return dispatch_c<128, In>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_cg_output(const CgOutputArgs& a, hipStream_t s) {
    return a.bf16 ? dispatch_d<bf16_t>(a, s) : dispatch_d<float>(a, s);
}

}  // namespace mesa
