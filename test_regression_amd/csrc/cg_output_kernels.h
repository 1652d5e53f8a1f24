// cg_output_kernels.h -- all CG iterations of one chunk plus the output
// contraction of the Mesa layer (gfx950): the kernels and their launch
// templates, instantiated by cg_output.hip (fp32 q/k/v, and bf16 at d = 16)
// and cg_output_bf16.hip (bf16 q/k/v at d >= 32).
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
// Work split: a workgroup works on one (head, chunk) at a time; wave w owns
// tokens 16w..16w+15 and runs their CG entirely on its own: the tiles in LDS
// are read-only during the iterations, so the CG loop has no workgroup
// barrier and waves stop independently.  Each wave runs a body specialised
// on w (static sub-chunk, causal block range).  The grid holds only as many
// workgroups as are resident at once (the LDS tiles allow one per compute
// unit at d = 128, C = 64), and each walks a strided list of chunks: the
// next chunk's stored state, keys, gates and queries are requested while
// the current chunk's output products run, instead of in a prologue that
// nothing overlaps.
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
#pragma once
#include <algorithm>
#include <atomic>

#include "cg_core.h"
#include "cg_h2.h"
#include "mesa_kernels.h"
#include "persistent.h"

namespace mesa {

// The query rows of the wave's tokens (B layout: lane (n, kk) holds features
// 16j + 4kk .. 16j + 4kk + 3 of token 16w + n), zero past the sequence end.
template <int D, typename In>
__device__ __forceinline__ void load_queries(Raw4<In> (&qr)[D / 16], const In* __restrict__ q, size_t tok0,
                                             int valid, int tr, int kk) {
#pragma unroll
    for (int j = 0; j < D / 16; ++j) {
        qr[j].zero();
        if (tr < valid) qr[j].load(q + (tok0 + tr) * D + 16 * j + 4 * kk);
    }
}

// One chunk's work of wave W (tokens 16W..16W+15): its CG, its output rows,
// and its share of loading and staging the next chunk of this workgroup.
// Four workgroup barriers: (A) every wave is done with the chunk's states,
// keys and gates; (B) V_c^T is staged; (C) the next chunk's S^H, K rows and
// gates are staged; (D) its K^T and mid-chunk state are formed.
template <int D, int C, int W, typename In>
__device__ __forceinline__ bool cg_wave(CgLds<D, C>& L, int tid, ChunkPos& p, int n_chunks, int H, int T,
                                        long total, int* __restrict__ work_counter, Raw4<In> (&qr)[D / 16],
                                        const In* __restrict__ q, const In* __restrict__ k,
                                        const In* __restrict__ v, const float* __restrict__ gamma,
                                        const float* __restrict__ lambda, const float* __restrict__ SH,
                                        const float* __restrict__ SG, int max_iters, float tol,
                                        float* __restrict__ out, int32_t* __restrict__ iters,
                                        float* __restrict__ x_out) {
    using CW = CgWave<D, C, W>;
    constexpr int NT = D / 16;
    constexpr int NW = C / 16;
    constexpr int NBO = CW::NBO;
    constexpr int NTHR = 64 * NW;
    constexpr int NLAM = (D + NTHR - 1) / NTHR;
    const int lane = tid & 63;
    const CW cw(L, lane);
    const int n = cw.n, kk = cw.kk, tr = cw.tr;
    const bool tok_ok = tr < p.valid;

    // ---- claim this workgroup's next chunk (its number arrives during the CG) ----
    int ticket = 0;
    if (W == 0 && lane == 0) ticket = atomicAdd(work_counter, 1);

    // ---- CG from x = 0 with r = p = q ----
    f32x4 X[NT], R[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) R[j] = qr[j].get();
    const int it = cg_solve_wave<D, C, W>(L, cw, R, X, max_iters, tol);
    // Addresses of the output phase are built from here on, not held across the CG.
    asm volatile("" : "+v"(tid));
    if (W == 0 && lane == 0) L.next = ticket;

    // ---- iteration counts, solutions ----
    if (iters && kk == 0 && tok_ok) iters[p.tok0 + tr] = it;
    if (x_out && tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j) store_row(x_out + (p.tok0 + tr) * D + 16 * j + 4 * kk, X[j]);
    }

    // ---- output O = diag(e^l) X G_c^T + (M o (X K^T)) V over the whole chunk, transposed ----
    // V_c is loaded into registers now and stored as V_c^T once every wave
    // is done with K_c^T; the state term takes G_c's blocks straight from
    // memory (stored in MFMA operand order: this lane's 16 bytes of block
    // (j, g) are G_c[16j + n][16g + 4kk .. 16g + 4kk + 3]), so it runs
    // before the barrier, while slower waves still iterate.
    ChunkRowsRegs<D, C, NTHR, In> vrows;
    vrows.load(v + p.tok0 * D, p.valid, tid);
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
    PackedStateRegs<D, NTHR> nsh;
    ChunkRowsRegs<D, C, NTHR, In> nk;
    float ngam = 1.0f, nlam[NLAM];
    f32x4 OS[NT], OI[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) OS[j] = OI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
        const float* gl = SG + p.soff + 4 * lane;
        constexpr int NB_G = 3;   // G_c block columns in flight: NB_G - 1 steps ahead
        f32x4 ga[NB_G][NT];
        auto gload = [&](int g, int buf) {
#pragma unroll
            for (int j = 0; j < NT; ++j) ga[buf][j] = *reinterpret_cast<const f32x4*>(gl + (j * NT + g) * 256);
        };
#pragma unroll
        for (int g = 0; g < NB_G - 1 && g < NT; ++g) gload(g, g);
#pragma unroll
        for (int g = 0; g < NT; ++g) {
            if (g + NB_G - 1 < NT) gload(g + NB_G - 1, (g + NB_G - 1) % NB_G);
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int j = 0; j < NT; ++j) OS[j] = mfma4(ga[g % NB_G][j][s], X[g][s], OS[j]);
        }
    }
    __syncthreads();   // (A) every wave is done with the states, K_c, K_c^T, l and lambda
    // Chunks 0..G-1 are the workgroups' first; the claims hand out the rest in order.
    const long nidx = (long)gridDim.x + __builtin_amdgcn_readfirstlane(L.next);
    const bool more = nidx < total;
    const ChunkPos pn = chunk_pos<D, C>(more ? nidx : 0, n_chunks, H, T);
    // The query registers are rewritten on every path (zero after the last
    // chunk), so their previous contents are dead once the CG has started.
    auto load_next = [&]() {
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
        load_queries<D, In>(qr, q, pn.tok0, more ? pn.valid : 0, tr, kk);
    };
    load_next();   // lands behind the V_c^T staging and the intra-chunk output products
    vrows.store_transposed(L.KT, tid);
    __syncthreads();   // (B)
    contract_intra<D, C, NBO, 0>(Wo, L.KT, n, kk, OI);
    if (tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] = cw.eLo * OS[j][r] + OI[j][r];
            store_row(out + (p.tok0 + tr) * D + 16 * j + 4 * kk, o);
        }
    }
    if (!more) return false;

    // ---- stage the next chunk ----
    nsh.store(L.R, tid);
    nk.store_rows(L.KV, tid);
    if (W == 0) {
        const float l = chunk_log_decay_of(ngam, pn.valid, lane);
        if (lane < C) L.L[lane] = l;
    }
#pragma unroll
    for (int u = 0; u < NLAM; ++u) {
        const int e = tid + u * NTHR;
        if (e < D) L.Lam[e] = nlam[u];
    }
    __syncthreads();   // (C) every wave is done with V_c^T
    nk.store_transposed(L.KT, tid);
    if constexpr (NW >= 2) form_mid_state<D, C>(L, W, n, kk);
    __syncthreads();   // (D)
    p = pn;
    return true;
}

// Persistent: G workgroups (as many as are resident at once) start on chunks
// 0..G-1 and then claim chunks G, G+1, ... in order from a counter (zeroed
// by the chunk-state kernel), so iteration counts that vary along the
// sequence still spread evenly; each chunk's state and key loads run behind
// the previous chunk's output products.
template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void cg_output_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ gamma, const float* __restrict__ lambda,
    const float* __restrict__ SH, const float* __restrict__ SG, int H, int T, int n_chunks, long total,
    int* __restrict__ work_counter, int max_iters, float tol, float* __restrict__ out, int32_t* __restrict__ iters,
    float* __restrict__ x_out) {
    constexpr int NW = C / 16;
    constexpr int NT = D / 16;
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
    Raw4<In> qr[NT];
    load_queries<D, In>(qr, q, p.tok0, p.valid, 16 * w + (lane & 15), lane >> 4);
    __syncthreads();
    if constexpr (NW >= 2) {
        form_mid_state<D, C>(L, w, lane & 15, lane >> 4);
        __syncthreads();
    }

    for (bool more = true; more;) {
        // An opaque copy of the thread id: the per-lane LDS addresses derived
        // from it are rebuilt per chunk instead of being held in registers
        // across the output phase.
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        if (w == 0) {
            more = cg_wave<D, C, 0, In>(L, tid, p, n_chunks, H, T, total, work_counter, qr, q, k, v, gamma, lambda,
                                        SH, SG, max_iters, tol, out, iters, x_out);
        } else if constexpr (NW > 1) {
            if (w == 1) {
                more = cg_wave<D, C, 1, In>(L, tid, p, n_chunks, H, T, total, work_counter, qr, q, k, v, gamma,
                                            lambda, SH, SG, max_iters, tol, out, iters, x_out);
            } else if constexpr (NW > 2) {
                if (w == 2)
                    more = cg_wave<D, C, 2, In>(L, tid, p, n_chunks, H, T, total, work_counter, qr, q, k, v, gamma,
                                                lambda, SH, SG, max_iters, tol, out, iters, x_out);
                else
                    more = cg_wave<D, C, 3, In>(L, tid, p, n_chunks, H, T, total, work_counter, qr, q, k, v, gamma,
                                                lambda, SH, SG, max_iters, tol, out, iters, x_out);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// d >= 32: the same persistent chunk loop with every matvec product on fp16
// MFMAs over two-part splits (cg_h2.h).  The chunk state is held whole (two
// fp16 planes of the full matrix).  Every wave's state term starts from
// S^H_c and its intra-chunk terms run over the causal keys from the chunk
// start, except at d = 128 with 64-token chunks and bf16 keys: there waves 2
// and 3 start their CG from the mid-chunk state (the state after token 31),
// which waves 0, 2 and 3 form at the chunk's start, so that their
// intra-chunk terms cover two key blocks at most, as wave 1's do.  Four
// workgroup barriers per chunk, as in cg_wave; the exponents of the next
// chunk's state and keys come from per-wave maxima gathered before barrier
// (C), and the values' exponent from maxima gathered before barrier (A).
// The output's V^T operands are read
// transposed from the value rows (staged where the key rows were, after
// barrier (A)), so the values need no transposed tile.
template <int D, int C, int W, typename In>
__device__ __forceinline__ bool cg_h2_wave(H2Lds<D, C, h2_key_planes<In>()>& L, uint32_t* Smid, uint32_t mc, int tid,
                                           ChunkPos& p, int& ES,
                                           int& EK, int n_chunks, int H, int T, long total,
                                           int* __restrict__ work_counter, Raw4<In> (&qr)[D / 16],
                                           const In* __restrict__ q, const In* __restrict__ k,
                                           const In* __restrict__ v, const float* __restrict__ gamma,
                                           const float* __restrict__ lambda, const float* __restrict__ SH,
                                           const float* __restrict__ SG, int max_iters, float tol,
                                           float* __restrict__ out, int32_t* __restrict__ iters,
                                           float* __restrict__ x_out) {
    constexpr int NKP = h2_key_planes<In>();
    using Wv = H2Wave<D, C, W>;
    constexpr int NT = D / 16;
    constexpr int NQ = D / 32;
    constexpr int NW = C / 16;
    constexpr int NTHR = 64 * NW;
    constexpr int NLAM = (D + NTHR - 1) / NTHR;
    const int lane = tid & 63;
    const Wv wv(L.L, lane);
    const int n = wv.n, kk = wv.kk, tr = wv.tr;
    const bool tok_ok = tr < p.valid;

    int ticket = 0;
    if (W == 0 && lane == 0) ticket = atomicAdd(work_counter, 1);

    // ---- CG from x = 0 with r = p = q ----
    f32x4 X[NT], R[NT], lam[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        R[j] = qr[j].get();
        lam[j] = lds4(&L.Lam[16 * j + 4 * kk]);   // held across the CG, off the update's path
    }
    int it;
    H2Hi<D, NKP> SHr;
    if constexpr (h2_mid_state<D, C, NKP>()) {
        // The mid-chunk state for waves 2 and 3, formed by waves 0, 2 and 3
        // (wave 1, with two key blocks from the chunk state, has no time to
        // spare), each a third of its 32 operand pieces: the lo parts into
        // Smid, the hi parts, once all four waves are done with the chunk
        // state's hi plane (count L.hand[0]), over that plane in L.S[0], where
        // waves 2 and 3 read the whole of it (count L.hand[1]).  Waves 0 and 1
        // take the chunk state's hi plane into registers first.
        constexpr int SW = H2Lds<D, C, NKP>::SW;
        constexpr int NP = NT * NQ;                         // operand pieces
        constexpr int F = W == 0 ? 0 : W == 1 ? -1 : W - 1;   // the wave's share, -1 none
        if constexpr (W < 2) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
#pragma unroll
                for (int i = 0; i < NT; ++i) SHr[q][i] = lds_f16x8(&L.S[0][(16 * i + n) * SW + 16 * q + 4 * kk]);
        }
        int EM = 0;
        if constexpr (F >= 0) {
            constexpr int PB = (NP * F + 2) / 3, PE = (NP * (F + 1) + 2) / 3;
            H2Hi<D, NKP> SM;
            EM = h2_form_mid<D, C, NKP, 2, PB, PE>(L, ES, EK, n, kk, Smid, SM);
            lds_signal(&L.hand[0], lane == 0);
            lds_wait_count(&L.hand[0], 4 * (mc + 1));
#pragma unroll
            for (int pc = PB; pc < PE; ++pc) {
                const int q = pc / NT, i = pc % NT;
                *reinterpret_cast<f16x8*>(&L.S[0][(16 * i + n) * SW + 16 * q + 4 * kk]) = SM[q][i];
            }
            lds_signal(&L.hand[1], lane == 0);
        } else {
            lds_signal(&L.hand[0], lane == 0);
        }
        if constexpr (W >= 2) {
            // waves 2 and 3: the state term from the mid-chunk state, keys
            // from block 2 on
            lds_wait_count(&L.hand[1], 3 * (mc + 1));
            const H2Wave<D, C, W, 2> wc(L.L, lane);
            // wave 3's lo plane through a register too (as waves 0-1's
            // below): the compiler's schedule of its loop then waits on its
            // LDS reads in pairs rather than one by one
            int o0 = 0;
            if constexpr (W == 3) asm volatile("" : "+v"(o0));
            it = h2_cg_solve<D, C, NKP, W, 2, false>(L, wc, EM, EK, R, X, lam, max_iters, tol, Smid + o0, SHr);
        } else {
            // the lo plane addressed through a register: with its constant
            // address the compiler waited on each of the loop's LDS reads
            // right after issuing it (wave 1: 28 full waits per iteration,
            // against 6 so, and 171k against 154k cycles per chunk for the CG)
            int o0 = 0;
            asm volatile("" : "+v"(o0));
            it = h2_cg_solve<D, C, NKP, W, 0, true>(L, wv, ES, EK, R, X, lam, max_iters, tol, L.S[1] + o0, SHr);
        }
    } else {
        it = h2_cg_solve<D, C, NKP, W, 0, false>(L, wv, ES, EK, R, X, lam, max_iters, tol, L.S[1], SHr);
    }
    asm volatile("" : "+v"(tid));
    if (W == 0 && lane == 0) L.next = ticket;

    if (iters && kk == 0 && tok_ok) iters[p.tok0 + tr] = it;
    if (x_out && tok_ok) {
#pragma unroll
        for (int j = 0; j < NT; ++j) store_row(x_out + (p.tok0 + tr) * D + 16 * j + 4 * kk, X[j]);
    }

    // ---- output O = diag(e^l) X G_c^T + (M o (X K^T)) V over the whole chunk, transposed ----
    // With at most two row blocks of G_c per wave (GL), the G_c term runs
    // after barrier (B) on fp16 MFMAs: each wave loads its row blocks of G_c
    // now, splits them after barrier (A) into two fp16 planes in the freed
    // state region (one exponent per row block), and after (B) every wave
    // reads them there.  Otherwise it streams the fp32 blocks onto fp32
    // MFMAs before (A).
    constexpr int RBW = (NT + NW - 1) / NW;   // row blocks of G_c a wave splits
    constexpr bool GL = RBW <= 2;
    const int g_row0 = W * RBW;
    f32x4 gr[GL ? RBW : 1][NT];
    if constexpr (GL) {
        const float* gl = SG + p.soff + 4 * lane;
#pragma unroll
        for (int i = 0; i < RBW; ++i)
#pragma unroll
            for (int g = 0; g < NT; ++g)
                gr[i][g] = g_row0 + i < NT ? *reinterpret_cast<const f32x4*>(gl + ((g_row0 + i) * NT + g) * 256)
                                           : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    ChunkRowsRegs<D, C, NTHR, In> vrows;
    vrows.load(v + p.tok0 * D, p.valid, tid);
    f32x4 Wo[2 * Wv::NS];
    const int EX = h2_exp(kslot_max(absmax<NT>(X)));
    f16x8 Xh[NQ], Xl[NQ];   // the solution's split, 2^EX
    {
        const float sX = pow2(EX);
        constexpr int NP = h2_score_parts<Wv::NBO, NKP>();
        f32x4 Sc[Wv::NBO][NP];
#pragma unroll
        for (int ib = 0; ib < Wv::NBO; ++ib)
#pragma unroll
            for (int t = 0; t < NP; ++t) Sc[ib][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) {
            h2_split(X[2 * qq], X[2 * qq + 1], sX, Xh[qq], Xl[qq]);
            h2_scores_step<D, C, NKP, Wv::NBO>(L, qq, Xh[qq], Xl[qq], n, kk, Sc);
        }
#pragma unroll
        for (int ib = 0; ib < 2 * Wv::NS; ++ib)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                Wo[ib][r] = ib < Wv::NBO ? h2_score<Wv::NBO, NKP>(Sc, ib < Wv::NBO ? ib : 0, r) * wv.dec[ib][r] : 0.f;
            }
    }
    PackedStateRegs<D, NTHR> nsh;
    ChunkRowsRegs<D, C, NTHR, In> nk;
    float ngam = 1.0f, nlam[NLAM];
    f32x4 OS[NT], OI[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) OS[j] = OI[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (!GL) {
        const float* gl = SG + p.soff + 4 * lane;
        constexpr int NB_G = 3;
        f32x4 ga[NB_G][NT];
        auto gload = [&](int g, int buf) {
#pragma unroll
            for (int j = 0; j < NT; ++j) ga[buf][j] = *reinterpret_cast<const f32x4*>(gl + (j * NT + g) * 256);
        };
#pragma unroll
        for (int g = 0; g < NB_G - 1 && g < NT; ++g) gload(g, g);
#pragma unroll
        for (int g = 0; g < NT; ++g) {
            if (g + NB_G - 1 < NT) gload(g + NB_G - 1, (g + NB_G - 1) % NB_G);
#pragma unroll
            for (int s2 = 0; s2 < 4; ++s2)
#pragma unroll
                for (int j = 0; j < NT; ++j) OS[j] = mfma4(ga[g % NB_G][j][s2], X[g][s2], OS[j]);
        }
    }
    {
        const float vm = wave_max(rows_absmax<D, C, NTHR, In>(vrows));
        if (lane == 0) L.red[2][W] = vm;
    }
    __syncthreads();   // (A) every wave is done with the state planes, K_c rows and K_c^T, l and lambda
    if constexpr (GL) {
        // the wave's row blocks of G_c as two fp16 planes where the state's were:
        // row 16 j + n, columns 16 g + 4 kk .. + 3 (perm32)
        constexpr int SW = H2Lds<D, C, NKP>::SW;
#pragma unroll
        for (int i = 0; i < RBW; ++i) {
            const int j = g_row0 + i;
            if (j < NT) {
                const int E = h2_exp(wave_max(absmax<NT>(gr[i])));
                const float sg = pow2(E);
#pragma unroll
                for (int g = 0; g < NT; ++g) {
                    f16x4 h, lo;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float y = gr[i][g][r] * sg;
                        h[r] = (_Float16)y;
                        lo[r] = (_Float16)(y - (float)h[r]);
                    }
                    const int w0 = (16 * j + n) * SW + perm32(16 * g + 4 * kk) / 2;
                    *reinterpret_cast<f16x4*>(&L.S[0][w0]) = h;
                    *reinterpret_cast<f16x4*>(&L.S[1][w0]) = lo;
                }
                if (lane == 0) L.gexp[j] = E;
            }
        }
    }
    float vmax = 0.f;
#pragma unroll
    for (int w2 = 0; w2 < NW; ++w2) vmax = fmaxf(vmax, L.red[2][w2]);
    const int EV = __builtin_amdgcn_readfirstlane(h2_exp(vmax));
    const long nidx = (long)gridDim.x + __builtin_amdgcn_readfirstlane(L.next);
    const bool more = nidx < total;
    const ChunkPos pn = chunk_pos<D, C>(more ? nidx : 0, n_chunks, H, T);
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
    load_queries<D, In>(qr, q, pn.tok0, more ? pn.valid : 0, tr, kk);
    stage_h2_rows<D, C, NTHR, NKP, In>(L.KR, vrows, tid, pow2(EV));   // V_c rows, where K_c's were
    __syncthreads();   // (B)
    if constexpr (GL) {
        // G_c X^T from the planes: three fp16 products per 32-feature step
        constexpr int SW = H2Lds<D, C, NKP>::SW;
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq)
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const int off = (16 * j + n) * SW + 16 * qq + 4 * kk;
                const f16x8 Gh = lds_f16x8(&L.S[0][off]), Gl = lds_f16x8(&L.S[1][off]);
                OS[j] = mfma_f16x32(Gl, Xh[qq], OS[j]);
                OS[j] = mfma_f16x32(Gh, Xl[qq], OS[j]);
                OS[j] = mfma_f16x32(Gh, Xh[qq], OS[j]);
            }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const float sj = pow2(-(L.gexp[j] + EX));
#pragma unroll
            for (int r = 0; r < 4; ++r) OS[j][r] *= sj;
        }
    }
    {
        const int EWo = h2_exp(kslot_max(absmax<2 * Wv::NS>(Wo)));
        h2_apply<D, C, NKP, Wv::NS>(L, Wo, pow2(EWo), n, kk, OI);
        const float bo = pow2(-(EV + EK + EX + EWo));
        if (tok_ok) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                f32x4 o;
#pragma unroll
                for (int r = 0; r < 4; ++r) o[r] = wv.eLo * OS[j][r] + bo * OI[j][r];
                store_row(out + (p.tok0 + tr) * D + 16 * j + 4 * kk, o);
            }
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
    __syncthreads();   // (C) every wave is done with V_c; the next chunk's maxima are in
    h2_stage_chunk<D, C, NTHR, NKP, In>(L, nsh, nk, tid, ES, EK);
    __syncthreads();   // (D)
    p = pn;
    return true;
}

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void cg_h2_kernel(
    const In* __restrict__ q, const In* __restrict__ k, const In* __restrict__ v,
    const float* __restrict__ gamma, const float* __restrict__ lambda,
    const float* __restrict__ SH, const float* __restrict__ SG, int H, int T, int n_chunks, long total,
    int* __restrict__ work_counter, int max_iters, float tol, float* __restrict__ out, int32_t* __restrict__ iters,
    float* __restrict__ x_out) {
    constexpr int NKP = h2_key_planes<In>();
    constexpr int NW = C / 16;
    constexpr int NT = D / 16;
    constexpr int NTHR = 64 * NW;
    __shared__ H2Lds<D, C, NKP> L;
    // the mid-chunk state's lo plane (waves 2 and 3 at d = 128, chunk 64, bf16
    // keys), on a 256-byte boundary as the chunk state's planes are (at 96
    // bytes past one, wave 3's iterations took 8% longer)
    __shared__ alignas(256) uint32_t Smid[h2_mid_state<D, C, NKP>() ? D * H2Lds<D, C, NKP>::SW : 4];

    const int tid0 = threadIdx.x;
    const int lane = tid0 & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    ChunkPos p = chunk_pos<D, C>(blockIdx.x, n_chunks, H, T);
    int ES, EK;

    // ---- the first chunk ----
    if constexpr (h2_mid_state<D, C, NKP>()) {
        // the hand-off counters, zeroed before the staging's barriers
        if (tid0 < 2) L.hand[tid0] = 0u;
    }
    h2_stage_first<D, C, NTHR, NKP, In>(L, p, SH, k, gamma, lambda, tid0, ES, EK);
    Raw4<In> qr[NT];
    load_queries<D, In>(qr, q, p.tok0, p.valid, 16 * w + (lane & 15), lane >> 4);

    uint32_t mc = 0;   // chunks this workgroup has taken before the current one
    for (bool more = true; more; ++mc) {
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        if (w == 0) {
            more = cg_h2_wave<D, C, 0, In>(L, Smid, mc, tid, p, ES, EK, n_chunks, H, T, total, work_counter, qr, q, k, v,
                                           gamma, lambda, SH, SG, max_iters, tol, out, iters, x_out);
        } else if constexpr (NW > 1) {
            if (w == 1) {
                more = cg_h2_wave<D, C, 1, In>(L, Smid, mc, tid, p, ES, EK, n_chunks, H, T, total, work_counter, qr, q, k,
                                               v, gamma, lambda, SH, SG, max_iters, tol, out, iters, x_out);
            } else if constexpr (NW > 2) {
                if (w == 2)
                    more = cg_h2_wave<D, C, 2, In>(L, Smid, mc, tid, p, ES, EK, n_chunks, H, T, total, work_counter, qr, q,
                                                   k, v, gamma, lambda, SH, SG, max_iters, tol, out, iters, x_out);
                else
                    more = cg_h2_wave<D, C, 3, In>(L, Smid, mc, tid, p, ES, EK, n_chunks, H, T, total, work_counter, qr, q,
                                                   k, v, gamma, lambda, SH, SG, max_iters, tol, out, iters, x_out);
            }
        }
    }
}

template <int D, int C, typename In>
static hipError_t launch_t(const CgOutputArgs& a, hipStream_t s) {
    if constexpr (D % 32 == 0) {
        static std::atomic<long> resident_h2[kMaxDevices];
        const long total = a.BH * a.n_chunks;
        const int block = 64 * (C / 16);
        const long grid = std::min(total, resident_workgroups(cg_h2_kernel<D, C, In>, block, resident_h2));
        hipLaunchKernelGGL((cg_h2_kernel<D, C, In>), dim3((unsigned)grid), dim3(block), 0, s,
                           (const In*)a.q, (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.SH, a.SG,
                           a.H, a.T, a.n_chunks, total, a.work_counter, a.max_iters, a.tol, a.out, a.iters,
                           a.x_out);
        return hipGetLastError();
    } else {
        static std::atomic<long> resident[kMaxDevices];
        const long total = a.BH * a.n_chunks;
        const int block = 64 * (C / 16);
        const long grid = std::min(total, resident_workgroups(cg_output_kernel<D, C, In>, block, resident));
        hipLaunchKernelGGL((cg_output_kernel<D, C, In>), dim3((unsigned)grid), dim3(block), 0, s,
                           (const In*)a.q, (const In*)a.k, (const In*)a.v, a.gamma, a.lambda, a.SH, a.SG,
                           a.H, a.T, a.n_chunks, total, a.work_counter, a.max_iters, a.tol, a.out, a.iters,
                           a.x_out);
        return hipGetLastError();
    }
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

}  // namespace mesa
