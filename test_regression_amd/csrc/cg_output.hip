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
// has no workgroup barrier and waves stop independently.  All contractions
// use v_mfma_f32_16x16x4_f32; the CG vectors x, r, p, y live in registers in
// MFMA accumulator layout, so the alpha/beta dot products are 16-lane DPP row
// reductions.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void cg_output_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ gamma, const float* __restrict__ lambda,
    const float* __restrict__ SH, const float* __restrict__ SGt, int H, int T, int n_chunks,
    int max_iters, float tol, float* __restrict__ out, int32_t* __restrict__ iters) {
    constexpr int NW = C / 16;   // waves per workgroup (16 tokens each)
    constexpr int NT = D / 16;   // 16-wide feature tiles
    constexpr int PD = lds_pitch(D);
    constexpr int PC = lds_pitch(C);
    constexpr int NTHR = 64 * NW;

    __shared__ float sS[D * PD];         // S^H_c, later (S^G_c)^T  [feature j][feature n]
    __shared__ float sKV[C * PD];        // K_c, later V_c          [token i][feature]
    __shared__ float sP[NW * 16 * PD];   // per wave: P (later X) rows, MFMA A staging
    __shared__ float sA[NW * 16 * PC];   // per wave: decayed scores M o (P K^T)
    __shared__ float sL[C];              // l_i
    __shared__ float sLam[D];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int n = lane & 15;
    const int kk = lane >> 4;

    const int c = blockIdx.x % n_chunks;
    const long bh = blockIdx.x / n_chunks;
    const int h = (int)(bh % H);
    const int t0 = c * C;
    const int valid = min(C, T - t0);

    const size_t tok0 = (size_t)bh * T + t0;   // first token of the chunk
    float* myP = sP + w * 16 * PD;
    float* myA = sA + w * 16 * PC;

    // ---------------- stage S^H_c, K_c, lambda, l ----------------
    {
        const float* src = SH + ((size_t)bh * n_chunks + c) * D * D;
        for (int e = tid * 4; e < D * D; e += NTHR * 4)
            *reinterpret_cast<f32x4*>(&sS[(e / D) * PD + e % D]) = *reinterpret_cast<const f32x4*>(src + e);
        for (int e = tid * 4; e < C * D; e += NTHR * 4) {
            const int i = e / D;
            f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < valid) x = load4(k + (tok0 + i) * D + e % D);
            *reinterpret_cast<f32x4*>(&sKV[i * PD + e % D]) = x;
        }
        for (int e = tid; e < D; e += NTHR) sLam[e] = lambda[(size_t)h * D + e];
        if (w == 0) {
            const float l = chunk_log_decay(gamma + tok0, valid, lane);
            if (lane < C) sL[lane] = l;
        }
    }
    __syncthreads();

    // ---------------- per-lane constants ----------------
    // lane rows: chunk-local token 16w + 4kk + r, r = 0..3; lane columns 16j + n
    float eL[4];
    float dec[NW][4];   // M[row][16ib + n]
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int tr = 16 * w + 4 * kk + r;
        eL[r] = __expf(sL[tr]);
#pragma unroll
        for (int ib = 0; ib < NW; ++ib) {
            const int i = 16 * ib + n;
            dec[ib][r] = (i <= tr) ? __expf(sL[tr] - sL[i]) : 0.f;
        }
    }
    float lamc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) lamc[j] = sLam[16 * j + n];

    // ---------------- CG state: x = 0, r = p = q ----------------
    f32x4 X[NT], R[NT], P[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * w + 4 * kk + r;
            R[j][r] = row < valid ? to_f32(q[(tok0 + row) * D + 16 * j + n]) : 0.f;
        }
        P[j] = R[j];
        X[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float rr[4], nq[4];
    bool done[4];
    int it[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        float s = 0.f;
#pragma unroll
        for (int j = 0; j < NT; ++j) s += R[j][r] * R[j][r];
        rr[r] = rowsum16(s);
        nq[r] = sqrtf(rr[r]);
        done[r] = !(rr[r] > 0.f);   // q_t == 0 (or a padded row): x = 0, 0 iterations
        it[r] = 0;
    }

    // Stage this wave's A operand rows (P or X) for the next contraction.
    auto stage_rows = [&](const f32x4 (&V)[NT]) {
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) myP[(4 * kk + r) * PD + 16 * j + n] = V[j][r];
        wave_lds_sync();
    };

    // Y = diag(e^l) Z sS + (M o (Z K^T)) sKV with Z the staged rows; the key
    // tile for the scores must be in sKV when this is called with K, and the
    // scores are kept in myA for the second (value) contraction.
    auto scores = [&]() {
        // One accumulator chain per 16-token key block, started inside its
        // own branch: no chain is ever carried (zero-initialised) across a
        // skipped block, which keeps every MFMA's accumulator input equal to
        // its output registers.
#pragma unroll
        for (int ib = 0; ib < NW; ++ib) {
            if (ib <= w) {
                f32x4 sc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int g = 0; g < NT; ++g) {
                    const f32x4 a4 = *reinterpret_cast<const f32x4*>(&myP[n * PD + 16 * g + 4 * kk]);
                    const f32x4 b4 = *reinterpret_cast<const f32x4*>(&sKV[(16 * ib + n) * PD + 16 * g + 4 * kk]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) sc = mfma4(a4[s], b4[s], sc);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r) myA[(4 * kk + r) * PC + 16 * ib + n] = sc[r] * dec[ib][r];
            }
        }
        wave_lds_sync();
    };
    auto state_term = [&](f32x4 (&Y)[NT]) {
#pragma unroll
        for (int j = 0; j < NT; ++j) Y[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < NT; ++g) {
            const f32x4 a4 = *reinterpret_cast<const f32x4*>(&myP[n * PD + 16 * g + 4 * kk]);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const float* brow = &sS[(16 * g + 4 * kk + s) * PD + n];
#pragma unroll
                for (int j = 0; j < NT; ++j) Y[j] = mfma4(a4[s], brow[16 * j], Y[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) Y[j][r] *= eL[r];
    };
    auto intra_term = [&](f32x4 (&Y)[NT]) {
#pragma unroll
        for (int ib = 0; ib < NW; ++ib) {
            if (ib <= w) {
                const f32x4 a4 = *reinterpret_cast<const f32x4*>(&myA[n * PC + 16 * ib + 4 * kk]);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const float* brow = &sKV[(16 * ib + 4 * kk + s) * PD + n];
#pragma unroll
                    for (int j = 0; j < NT; ++j) Y[j] = mfma4(a4[s], brow[16 * j], Y[j]);
                }
            }
        }
    };

    stage_rows(P);

    // ---------------- CG iterations ----------------
    for (int itn = 0; itn < max_iters; ++itn) {
        bool alive = false;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            if (!done[r]) {
                const float rho = sqrtf(rr[r]) / nq[r];
                if ((tol > 0.f && rho < tol) || rr[r] == 0.f) done[r] = true;
                else alive = true;
            }
        }
        if (__builtin_amdgcn_ballot_w64(alive) == 0) break;

        f32x4 Y[NT];
        state_term(Y);
        scores();
        intra_term(Y);
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) Y[j][r] += lamc[j] * P[j][r];

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
        stage_rows(P);
    }

    // ---------------- iteration counts ----------------
    if (iters && n == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * w + 4 * kk + r;
            if (row < valid) iters[tok0 + row] = it[r];
        }
    }

    // ---------------- output O = G_t x ----------------
    stage_rows(X);
    scores();            // M o (X K^T), still against the keys
    __syncthreads();     // every wave is done with S^H_c and K_c
    {
        const float* src = SGt + ((size_t)bh * n_chunks + c) * D * D;
        for (int e = tid * 4; e < D * D; e += NTHR * 4)
            *reinterpret_cast<f32x4*>(&sS[(e / D) * PD + e % D]) = *reinterpret_cast<const f32x4*>(src + e);
        for (int e = tid * 4; e < C * D; e += NTHR * 4) {
            const int i = e / D;
            f32x4 x = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < valid) x = load4(v + (tok0 + i) * D + e % D);
            *reinterpret_cast<f32x4*>(&sKV[i * PD + e % D]) = x;
        }
    }
    __syncthreads();
    f32x4 O[NT];
    state_term(O);
    intra_term(O);
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * w + 4 * kk + r;
            if (row < valid) out[(tok0 + row) * D + 16 * j + n] = O[j][r];
        }
}

template <int D, int C, typename In>
static hipError_t launch_t(const CgOutputArgs& a, hipStream_t s) {
    const long grid = a.BH * a.n_chunks;
    hipLaunchKernelGGL((cg_output_kernel<D, C, In>), dim3((unsigned)grid), dim3(64 * (C / 16)), 0, s,
                       (const In*)a.q, (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.SH, a.SGt,
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
