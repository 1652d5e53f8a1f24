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
#include "cg_core.h"
#include "mesa_kernels.h"

namespace mesa {

// The CG of wave W (tokens 16W..16W+15 of the chunk) and its output rows.
template <int D, int C, int W, typename In>
__device__ __forceinline__ void cg_wave(CgLds<D, C>& L, int tid, const In* __restrict__ q,
                                        const In* __restrict__ v, const float* __restrict__ Gc, size_t tok0,
                                        int valid, int max_iters, float tol, float* __restrict__ out,
                                        int32_t* __restrict__ iters, float* __restrict__ x_out) {
    using CW = CgWave<D, C, W>;
    constexpr int NT = D / 16;
    constexpr int NW = C / 16;
    constexpr int NBO = CW::NBO;
    constexpr int NTHR = 64 * NW;
    const CW cw(L, tid & 63);
    const int n = cw.n, kk = cw.kk, tr = cw.tr;
    const bool tok_ok = tr < valid;

    // ---- CG from x = 0 with r = p = q ----
    f32x4 X[NT], R[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j)
        R[j] = tok_ok ? load4(q + (tok0 + tr) * D + 16 * j + 4 * kk) : f32x4{0.f, 0.f, 0.f, 0.f};
    const int it = cg_solve_wave<D, C, W>(L, cw, R, X, max_iters, tol);

    // ---- iteration counts, solutions ----
    if (iters && kk == 0 && tok_ok) iters[tok0 + tr] = it;
    if (x_out && tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j) *reinterpret_cast<f32x4*>(x_out + (tok0 + tr) * D + 16 * j + 4 * kk) = X[j];
    }

    // ---- output O = diag(e^l) X G_c^T + (M o (X K^T)) V over the whole chunk, transposed ----
    // V_c is loaded into registers now and stored as V_c^T once every wave
    // is done with K_c^T; the state term takes G_c's blocks straight from
    // memory (stored in MFMA operand order: this lane's 16 bytes of block
    // (j, g) are G_c[16j + n][16g + 4kk .. 16g + 4kk + 3]), so it runs
    // before the barrier, while slower waves still iterate.
    ChunkRowsRegs<D, C, NTHR, In> vrows;
    vrows.load(v + tok0 * D, valid, tid);
    f32x4 Wo[NBO];
    {
        f32x4 Sc[NBO], unused[NT];
#pragma unroll
        for (int ib = 0; ib < NBO; ++ib) Sc[ib] = f32x4{0.f, 0.f, 0.f, 0.f};
        contract_rows<D, NBO, false>(X, nullptr, L.KV, n, kk, unused, Sc);
#pragma unroll
        for (int ib = 0; ib < NBO; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) Wo[ib][r] = Sc[ib][r] * cw.dec[ib][r];
    }
    f32x4 OS[NT], OI[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) OS[j] = OI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const float* gl = Gc + 4 * (tid & 63);
        f32x4 ga[3][NT];
        auto gload = [&](int g, int buf) {
#pragma unroll
            for (int j = 0; j < NT; ++j) ga[buf][j] = *reinterpret_cast<const f32x4*>(gl + (j * NT + g) * 256);
        };
        gload(0, 0);
        if (NT > 1) gload(1, 1);
#pragma unroll
        for (int g = 0; g < NT; ++g) {
            if (g + 2 < NT) gload(g + 2, (g + 2) % 3);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int j = 0; j < NT; ++j) OS[j] = mfma4(ga[g % 3][j][s], X[g][s], OS[j]);
        }
    }
    __syncthreads();   // every wave is done with the states, K_c and K_c^T
    vrows.store_transposed(L.KT, tid);
    __syncthreads();
    contract_intra<D, C, NBO, 0>(Wo, L.KT, n, kk, OI);
    if (tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = cw.eLo * OS[j][r] + OI[j][r];
            *reinterpret_cast<f32x4*>(out + (tok0 + tr) * D + 16 * j + 4 * kk) = o;
        }
    }
}

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void cg_output_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ gamma, const float* __restrict__ lambda,
    const float* __restrict__ SH, const float* __restrict__ SG, int H, int T, int n_chunks,
    int max_iters, float tol, float* __restrict__ out, int32_t* __restrict__ iters, float* __restrict__ x_out) {
    constexpr int NW = C / 16;
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

    // ---- stage S^H_c, K_c (rows and transposed), lambda, l ----
    stage_packed_state<D, C>(L, SH + hoff, tid, NTHR);
    stage_chunk_rows<D, C, true, true>(L.KV, L.KT, k + tok0 * D, valid, tid, NTHR);
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
        cg_wave<D, C, 0, In>(L, tid, q, v, Gc, tok0, valid, max_iters, tol, out, iters, x_out);
    } else if constexpr (NW > 1) {
        if (w == 1) {
            cg_wave<D, C, 1, In>(L, tid, q, v, Gc, tok0, valid, max_iters, tol, out, iters, x_out);
        } else if constexpr (NW > 2) {
            if (w == 2) cg_wave<D, C, 2, In>(L, tid, q, v, Gc, tok0, valid, max_iters, tol, out, iters, x_out);
            else cg_wave<D, C, 3, In>(L, tid, q, v, Gc, tok0, valid, max_iters, tol, out, iters, x_out);
        }
    }
}

template <int D, int C, typename In>
static hipError_t launch_t(const CgOutputArgs& a, hipStream_t s) {
    const long grid = a.BH * a.n_chunks;
    hipLaunchKernelGGL((cg_output_kernel<D, C, In>), dim3((unsigned)grid), dim3(64 * (C / 16)), 0, s,
                       (const In*)a.q, (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.SH, a.SG,
                       a.H, a.T, a.n_chunks, a.max_iters, a.tol, a.out, a.iters, a.x_out);
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
