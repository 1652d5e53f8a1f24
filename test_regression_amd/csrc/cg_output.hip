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
// Chunkwise form used here (chunk c covers tokens t0..t0+C-1, l_t the
// within-chunk prefix sum of ln gamma, S^H_c = H_{t0-1}, S^G_c = G_{t0-1}):
//   H_t p = e^{l_t} S^H_c p + sum_{i=t0..t} e^{l_t - l_i} (k_i . p) k_i
//   G_t x = e^{l_t} S^G_c x + sum_{i=t0..t} e^{l_t - l_i} (k_i . x) v_i
// For the C tokens of a chunk at once (P, K, V in R^{C x d},
// M_ti = e^{l_t - l_i} [i <= t]):
//   Y = diag(e^l) P S^H_c + (M o (P K^T)) K + P diag(lambda)
//   O = diag(e^l) X (S^G_c)^T + (M o (X K^T)) V
// The keys are both the "keys" and the "values" of the CG matvec and do not
// change between iterations, so S^H_c and K_c stay in LDS for every
// iteration.
//
// Work split: one workgroup per (head, chunk); wave w owns tokens
// 16w..16w+15 of the chunk and runs their CG entirely on its own: the state
// and key tiles in LDS are read-only during the iterations, so the CG loop
// has no workgroup barrier and waves stop independently.  Each wave runs a
// body specialised on w, so its causal block count (w + 1 key blocks) is a
// compile-time constant.  All contractions use v_mfma_f32_16x16x4_f32; the
// CG vectors x, r, p, y live in registers in MFMA accumulator layout, so the
// alpha/beta dot products are 16-lane DPP row reductions.
//
// Operand loads: the contraction index of every MFMA is mapped so that a
// lane's four k-values are contiguous, and every B operand that is a matrix
// row in LDS (S^H, which is symmetric; G, stored row-major; the key rows of
// the scores) is read 128 bits at a time.  The next k-group's operands are
// loaded before the current group's MFMAs are issued: with one wave per
// SIMD (the tiles take ~150 KiB of LDS) the wave hides its own LDS latency.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

template <int D, int C>
struct CgLds {
    static constexpr int NW = C / 16;
    static constexpr int PD = lds_pitch(D);
    static constexpr int PS = lds_pitch_rows(D);
    static constexpr int PC = lds_pitch(C);
    float S[D * PS];          // S^H_c, later G_c           [row][feature]
    float KV[C * PD];         // K_c, later V_c             [token][feature]
    float P[NW][16 * PD];     // per wave: P (later X) rows, MFMA A staging
    float A[NW][16 * PC];     // per wave: decayed scores M o (Z K^T)
    float L[C];               // l_i
    float Lam[D];
};

__device__ __forceinline__ f32x4 lds4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Y[j]  += sum_f Z[m][f] * Bs[16j + n][f]      (if STATE; Bs symmetric or row-major G)
// Sc[ib] += sum_f Z[m][f] * Bk[16ib + n][f]    (ib < NB; the score blocks)
// Z, Bk: LDS rows of pitch lds_pitch(D); Bs: pitch lds_pitch_rows(D).  Software-pipelined over the
// 16-wide k-groups: group g+1's operands are in flight while group g's MFMAs
// issue.
template <int D, int NB, bool STATE>
__device__ __forceinline__ void contract_rows(const float* Z, const float* Bs, const float* Bk, int n, int kk,
                                              f32x4 (&Y)[D / 16], f32x4 (&Sc)[NB > 0 ? NB : 1]) {
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    constexpr int PS = lds_pitch_rows(D);
    constexpr int NBB = NB > 0 ? NB : 1;
    const float* za = Z + n * PD + 4 * kk;
    const float* bsa = STATE ? Bs + n * PS + 4 * kk : nullptr;
    const float* bka = NB > 0 ? Bk + n * PD + 4 * kk : nullptr;
    f32x4 a[2], bs[2][STATE ? NT : 1], bk[2][NBB];
    auto load = [&](int g, int buf) {
        a[buf] = lds4(za + 16 * g);
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
                for (int j = 0; j < NT; ++j) Y[j] = mfma4(a[cur][s], bs[cur][j][s], Y[j]);
            }
#pragma unroll
            for (int ib = 0; ib < NB; ++ib) Sc[ib] = mfma4(a[cur][s], bk[cur][ib][s], Sc[ib]);
        }
    }
}

// Y[j] += sum_{i < 16 NB} A[m][i] * B[i][16j + n]   (A: per-wave scores,
// pitch lds_pitch(C); B: K or V tile rows, pitch lds_pitch(D)).
template <int D, int C, int NB>
__device__ __forceinline__ void contract_intra(const float* A, const float* B, int n, int kk, f32x4 (&Y)[D / 16]) {
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    constexpr int PC = lds_pitch(C);
    float b[2][NT];
    auto load = [&](int ib, int s, int buf) {
        const float* brow = B + (16 * ib + 4 * kk + s) * PD + n;
#pragma unroll
        for (int j = 0; j < NT; ++j) b[buf][j] = brow[16 * j];
    };
    load(0, 0, 0);
#pragma unroll
    for (int ib = 0; ib < NB; ++ib) {
        const f32x4 a4 = lds4(A + n * PC + 16 * ib + 4 * kk);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int step = 4 * ib + s, cur = step & 1;
            if (step + 1 < 4 * NB) load((step + 1) / 4, (step + 1) % 4, cur ^ 1);
#pragma unroll
            for (int j = 0; j < NT; ++j) Y[j] = mfma4(a4[s], b[cur][j], Y[j]);
        }
    }
}

// Stage a wave's 16 rows (MFMA accumulator layout) as A-operand rows in LDS.
template <int D>
__device__ __forceinline__ void stage_rows(float* dst, const f32x4 (&V)[D / 16], int n, int kk) {
    constexpr int PD = lds_pitch(D);
#pragma unroll
    for (int j = 0; j < D / 16; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * kk + r) * PD + 16 * j + n] = V[j][r];
    wave_lds_sync();
}

template <int C, int NB>
__device__ __forceinline__ void stage_scores(float* dst, const f32x4 (&Sc)[NB], const float (&dec)[NB][4], int n,
                                             int kk) {
    constexpr int PC = lds_pitch(C);
#pragma unroll
    for (int ib = 0; ib < NB; ++ib)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(4 * kk + r) * PC + 16 * ib + n] = Sc[ib][r] * dec[ib][r];
    wave_lds_sync();
}

// The CG of wave W (tokens 16W..16W+15 of the chunk) and its output rows.
template <int D, int C, int W, typename In>
__device__ __forceinline__ void cg_wave(CgLds<D, C>& L, int tid, const In* __restrict__ q,
                                        const In* __restrict__ v, const float* __restrict__ Gc, size_t tok0,
                                        int valid, int max_iters, float tol, float* __restrict__ out,
                                        int32_t* __restrict__ iters) {
    constexpr int NT = D / 16;
    constexpr int NB = W + 1;          // causal key blocks of this wave
    constexpr int PD = lds_pitch(D);
    constexpr int PS = lds_pitch_rows(D);
    constexpr int NTHR = 64 * (C / 16);
    const int lane = tid & 63;
    const int n = lane & 15;
    const int kk = lane >> 4;
    float* myP = L.P[W];
    float* myA = L.A[W];

    // ---- per-lane constants; lane rows are chunk tokens 16W + 4kk + r ----
    float eL[4];
    float dec[NB][4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tr = 16 * W + 4 * kk + r;
        eL[r] = __expf(L.L[tr]);
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) {
            const int i = 16 * ib + n;
            dec[ib][r] = (i <= tr) ? __expf(L.L[tr] - L.L[i]) : 0.f;
        }
    }
    float lamc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) lamc[j] = L.Lam[16 * j + n];

    // ---- CG state: x = 0, r = p = q ----
    f32x4 X[NT], R[NT], P[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * W + 4 * kk + r;
            R[j][r] = row < valid ? to_f32(q[(tok0 + row) * D + 16 * j + n]) : 0.f;
        }
        P[j] = R[j];
        X[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // stop before an update when |r| / |q| < tol, tested as r.r < (tol |q|)^2
    float rr[4], stop_rr[4];
    bool done[4];
    int it[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j) s += R[j][r] * R[j][r];
        rr[r] = rowsum16(s);
        const float tq = tol * sqrtf(rr[r]);
        stop_rr[r] = tq * tq;
        done[r] = !(rr[r] > 0.f);   // q_t == 0 (or a padded row): x = 0, 0 iterations
        it[r] = 0;
    }
    stage_rows<D>(myP, P, n, kk);

    // ---- CG iterations ----
    for (int itn = 0; itn < max_iters; ++itn) {
        bool alive = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!done[r]) {
                if (rr[r] < stop_rr[r] || rr[r] == 0.f) done[r] = true;
                else alive = true;
            }
        }
        if (__builtin_amdgcn_ballot_w64(alive) == 0) break;

        // Y = diag(e^l) P S^H + (M o (P K^T)) K + diag(lambda) P.  Each MFMA
        // chain starts from zero and is only read afterwards (never written
        // back into), so the state and intra-chunk sums use separate
        // accumulators and are combined on the VALU.
        f32x4 Y[NT];
        {
            f32x4 YS[NT], YI[NT], Sc[NB];
#pragma unroll
            for (int j = 0; j < NT; ++j) YS[j] = YI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ib = 0; ib < NB; ++ib) Sc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
            contract_rows<D, NB, true>(myP, L.S, L.KV, n, kk, YS, Sc);
            stage_scores<C, NB>(myA, Sc, dec, n, kk);
            contract_intra<D, C, NB>(myA, L.KV, n, kk, YI);
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) Y[j][r] = eL[r] * YS[j][r] + YI[j][r] + lamc[j] * P[j][r];
        }

        float alpha[4];
        bool act[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < NT; ++j) s += P[j][r] * Y[j][r];
            const float pap = rowsum16(s);
            act[r] = !done[r] && (pap > 0.f);
            if (!done[r] && !act[r]) done[r] = true;   // breakdown guard
            alpha[r] = act[r] ? rr[r] / pap : 0.f;
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                X[j][r] += alpha[r] * P[j][r];
                R[j][r] -= alpha[r] * Y[j][r];
            }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float s = 0.f;
#pragma unroll
            for (int j = 0; j < NT; ++j) s += R[j][r] * R[j][r];
            const float rrn = rowsum16(s);
            if (act[r]) {
                const float beta = rrn / rr[r];
#pragma unroll
                for (int j = 0; j < NT; ++j) P[j][r] = R[j][r] + beta * P[j][r];
                rr[r] = rrn;
                it[r] += 1;
            }
        }
        stage_rows<D>(myP, P, n, kk);
    }

    // ---- iteration counts ----
    if (iters && n == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * W + 4 * kk + r;
            if (row < valid) iters[tok0 + row] = it[r];
        }
    }

    // ---- output O = diag(e^l) X G_c^T + (M o (X K^T)) V ----
    stage_rows<D>(myP, X, n, kk);
    {
        f32x4 unused[NT], Sc[NB];
#pragma unroll
        for (int ib = 0; ib < NB; ++ib) Sc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        contract_rows<D, NB, false>(myP, nullptr, L.KV, n, kk, unused, Sc);
        stage_scores<C, NB>(myA, Sc, dec, n, kk);
    }
    __syncthreads();   // every wave is done with S^H_c and K_c
    for (int e = tid * 4; e < D * D; e += NTHR * 4)
        *reinterpret_cast<f32x4*>(&L.S[(e / D) * PS + e % D]) = *reinterpret_cast<const f32x4*>(Gc + e);
    for (int e = tid * 4; e < C * D; e += NTHR * 4) {
        const int i = e / D;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i < valid) x = load4(v + (tok0 + i) * D + e % D);
        *reinterpret_cast<f32x4*>(&L.KV[i * PD + e % D]) = x;
    }
    __syncthreads();
    f32x4 OS[NT], OI[NT], none[1];
#pragma unroll
    for (int j = 0; j < NT; ++j) OS[j] = OI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    contract_rows<D, 0, true>(myP, L.S, nullptr, n, kk, OS, none);
    contract_intra<D, C, NB>(myA, L.KV, n, kk, OI);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * W + 4 * kk + r;
            if (row < valid) out[(tok0 + row) * D + 16 * j + n] = eL[r] * OS[j][r] + OI[j][r];
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
    const size_t tok0 = (size_t)bh * T + t0;   // first token of the chunk
    const size_t soff = ((size_t)bh * n_chunks + c) * D * D;

    // ---- stage S^H_c, K_c, lambda, l ----
    for (int e = tid * 4; e < D * D; e += NTHR * 4)
        *reinterpret_cast<f32x4*>(&L.S[(e / D) * PS + e % D]) = *reinterpret_cast<const f32x4*>(SH + soff + e);
    for (int e = tid * 4; e < C * D; e += NTHR * 4) {
        const int i = e / D;
        f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i < valid) x = load4(k + (tok0 + i) * D + e % D);
        *reinterpret_cast<f32x4*>(&L.KV[i * PD + e % D]) = x;
    }
    for (int e = tid; e < D; e += NTHR) L.Lam[e] = lambda[(size_t)h * D + e];
    if (w == 0) {
        const float l = chunk_log_decay(gamma + tok0, valid, lane);
        if (lane < C) L.L[lane] = l;
    }
    __syncthreads();

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
