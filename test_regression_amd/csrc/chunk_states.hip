// chunk_states.hip -- chunk-boundary states of the Mesa layer (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section "A Camada
// Mesa", bullet "Paralelizacao": the layer keeps the state variables H_t and
// G_t and solves chunks of the sequence in parallel.  With the forget factors
// zeta_{tt'} = prod_{s=t'+1..t} gamma_s the states obey
//   H_t = gamma_t H_{t-1} + k_t k_t^T,   G_t = gamma_t G_{t-1} + v_t k_t^T.
// Over a chunk c of C tokens with within-chunk log decays l_i (prefix sums of
// ln gamma) this is
//   S_{c+1} = e^{l_end} S_c + sum_{i in c} e^{l_end - l_i} a_i k_i^T,
// a = k for H and a = v for G, S_0 = 0.  This kernel produces S_c for every
// chunk (the state before the chunk's first token) and, optionally, the final
// state after the last token.
//
// Chunk states in the workspace: G as all its 16 x 16 blocks, H (symmetric)
// as the upper triangle of them -- the part the CG kernel reads -- each in
// row-major block order, so a wave stores a block as one 16-byte piece per
// lane (1 KiB contiguous per wave).  An H block is kept in MFMA accumulator
// order (lane 16q + m holds rows 4q..4q+3 of column m); a G block in MFMA
// operand order (lane 16q + m holds columns 4q..4q+3 of row m), which is the
// A operand the CG kernel's output product takes straight from memory.  For
// the backward's adjoint solve (g_transposed) the blocks of G^T are stored
// in operand order instead, the A operand of its G^T g product.  The
// exported final states are full and row-major ([d_v][d_k] for G).
//
// Work split: one workgroup per (head, {H, G}, 16*NW-row block of the
// state); each wave holds a 16 x D slab of the running state (of H, or of
// G^T: 16 key features by all value features) in MFMA accumulator layout
// and walks the chunks in order.  Per chunk the update is one
// (16 x C) x (C x D) product on v_mfma_f32_16x16x4_f32 with the weighted keys
// as the A operand and the keys (H) or values (G^T) as the B operand; the
// contraction runs over the chunk's tokens.  For bf16 keys and values the
// product runs on v_mfma_f32_16x16x32_bf16 instead: the values a_i, b_i are
// exact bf16, and each weighted value w_i a_i (a float) is split exactly into
// three bf16 parts (the top 8, next 8 and last 8 bits of its significand),
// so the three bf16 products sum to the float product terms up to the
// accumulation order.  The chunk's values are then staged as bf16 with two
// consecutive tokens per 32-bit LDS word, so a lane's eight-token MFMA
// operand is four word reads.  Workgroup ids are
// mapped so that the 2*RB workgroups of one head land on the same XCD (ids
// congruent mod 8) and share its L2 for the key and value tiles.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

// Offset (floats) of block (a, b), a <= b, in the packed upper block triangle
// of a d x d state (16 x 16 blocks stored row-major one after another).
template <int NT>
__device__ __forceinline__ int packed_blk(int a, int b) {
    return (a * NT - a * (a - 1) / 2 + (b - a)) * 256;
}

// NWK: waves per workgroup (each owns 16 rows of the state).  With
// NWK = D / 16 a workgroup holds a whole state (one per head for H, one for
// G); fewer waves split a state into RB row blocks, giving more workgroups
// for problems with few heads.
template <int D, int C, int NWK, typename In>
__global__ __launch_bounds__(64 * NWK) void chunk_states_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma,
    int T, int n_chunks, float* __restrict__ SH, float* __restrict__ SG,
    float* __restrict__ final_H, float* __restrict__ final_G, int write_chunks, long BH,
    int* __restrict__ work_counter, int g_transposed) {
    constexpr int NW = NWK;                    // waves per workgroup
    constexpr int RB = D / (16 * NW);          // row blocks per state
    constexpr int NT = D / 16;                 // 16-column tiles of the state
    constexpr int PD = lds_pitch(D);
    constexpr int NTHR = 64 * NW;
    constexpr int HPACK = D * (D + 16) / 2;    // floats of a packed upper block triangle
    constexpr bool BF = sizeof(In) == 2;       // bf16 keys and values: the split bf16 product
    // bf16 tiles: word (p, f) holds feature f of tokens 2p (low half) and
    // 2p + 1 (high half); the pitch D + 8 puts the four lane groups' rows
    // (2 token pairs apart) 16 banks apart.
    constexpr int PP = D + 8;
    constexpr int TILE = BF ? (C / 2) * PP : C * PD;

    __shared__ float sK[TILE];     // keys of the chunk (A operand; B operand for H)
    __shared__ float sB[TILE];     // values of the chunk (B operand for G^T)
    __shared__ alignas(16) float sW[C];   // e^{l_end - l_i}
    __shared__ float sGam;         // e^{l_end}

    const int tid0 = threadIdx.x;
    const int lane = tid0 & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int n = lane & 15;
    const int kk = lane >> 4;
    // the chunk-claim counter of the CG/output kernel that runs next
    if (work_counter && blockIdx.x == 0 && tid0 == 0) *work_counter = 0;

    // XCD-aware id: consecutive ids go round-robin over the 8 XCDs, so the
    // 2*RB parts of head bh get ids xcd + 8*(slot) with equal xcd.
    constexpr int PARTS = 2 * RB;
    const long xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const long bh = (slot / PARTS) * 8 + xcd;
    const int part = (int)(slot % PARTS);
    if (bh >= BH) return;                      // whole workgroup: no barrier is skipped
    const int rb = part % RB;
    const int which = part / RB;               // 0: H, 1: G
    const int m0 = rb * 16 * NW + 16 * w;      // first state row (of H or G^T) of this wave
    const int a0 = m0 / 16;                    // its row block

    const In* kh = k + (size_t)bh * T * D;
    const In* vh = v + (size_t)bh * T * D;
    const float* gh = gamma + (size_t)bh * T;
    // H: packed upper block triangle per chunk; G: full d x d per chunk
    float* Sout = which == 0 ? SH + (size_t)bh * n_chunks * HPACK : SG + (size_t)bh * n_chunks * D * D;
    // H: A = weighted keys, B = keys.  G: the wave's slab is of G^T (A =
    // weighted keys, B = values), whose accumulator blocks are G's blocks in
    // operand order; with g_transposed, of G (A = weighted values, B = keys),
    // whose accumulator blocks are G^T's blocks in operand order.
    const bool gt = which == 1 && g_transposed;
    const float* sArows = gt ? sB : sK;
    const float* sBcols = which == 0 || gt ? sK : sB;

    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Keys, values and gates of the next RING chunks are held in registers
    // (a ring of RING slots), so a chunk's global loads have RING chunk
    // steps of MFMAs and stores to complete behind.  Two slots of fp32
    // inputs would cost the second wave per SIMD its registers.
    constexpr int RING = sizeof(In) == 2 ? 2 : 1;
    constexpr int EL4 = C * D / (4 * NTHR);   // 4-element groups per thread per tile
    static_assert(C * D % (4 * NTHR) == 0, "tile must split evenly over the workgroup");
    Raw4<In> kreg[RING][EL4], vreg[RING][EL4];
    float greg[RING];
#pragma unroll
    for (int sl = 0; sl < RING; ++sl) greg[sl] = 1.0f;
    // Lane-dependent addresses are rebuilt from an opaque copy of the thread
    // id in every step and prefetch instead of being held in registers
    // across the chunk loop (which would cost the second wave per SIMD).
    auto prefetch = [&](int c, int sl) {
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int t0 = c * C;
        const int valid = min(C, T - t0);
#pragma unroll
        for (int u = 0; u < EL4; ++u) {
            const int e = (tid + u * NTHR) * 4;
            const int i = e / D, f = e % D;
            kreg[sl][u].zero();
            vreg[sl][u].zero();
            if (i < valid) {
                kreg[sl][u].load(kh + (size_t)(t0 + i) * D + f);
                if (which) vreg[sl][u].load(vh + (size_t)(t0 + i) * D + f);
            }
        }
        if (w == 0) greg[sl] = lane < valid ? gh[t0 + lane] : 1.0f;
    };

    auto step = [&](int c, int sl) {
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, n = lane & 15, kk = lane >> 4;
        // ---- stage the chunk's keys (and values) in LDS ----
#pragma unroll
        for (int u = 0; u < EL4; ++u) {
            const int e = (tid + u * NTHR) * 4;
            const int i = e / D, f = e % D;
            if constexpr (BF) {
                uint16_t* k16 = reinterpret_cast<uint16_t*>(sK) + ((i >> 1) * PP + f) * 2 + (i & 1);
                uint16_t* v16 = reinterpret_cast<uint16_t*>(sB) + ((i >> 1) * PP + f) * 2 + (i & 1);
                const uint2 kb = kreg[sl][u].raw(), vb = vreg[sl][u].raw();
                k16[0] = (uint16_t)kb.x;
                k16[2] = (uint16_t)(kb.x >> 16);
                k16[4] = (uint16_t)kb.y;
                k16[6] = (uint16_t)(kb.y >> 16);
                if (which) {
                    v16[0] = (uint16_t)vb.x;
                    v16[2] = (uint16_t)(vb.x >> 16);
                    v16[4] = (uint16_t)vb.y;
                    v16[6] = (uint16_t)(vb.y >> 16);
                }
            } else {
                *reinterpret_cast<f32x4*>(&sK[i * PD + f]) = kreg[sl][u].get();
                if (which) *reinterpret_cast<f32x4*>(&sB[i * PD + f]) = vreg[sl][u].get();
            }
        }
        if (w == 0) {
            // within-chunk log decays (tokens past the end count as gamma = 1)
            float l = __logf(greg[sl]);
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const float t = __shfl_up(l, o, 64);
                if (lane >= o) l += t;
            }
            const float lend = __shfl(l, C - 1, 64);
            if (lane < C) sW[lane] = __expf(lend - l);
            if (lane == 0) sGam = __expf(lend);
        }
        __syncthreads();
        if (c + RING < n_chunks) prefetch(c + RING, sl);

        // ---- the state before this chunk ----
        if (write_chunks) {
            // one 16-byte piece per lane per 16 x 16 block (accumulator order)
            float* dst = Sout + (size_t)c * (which == 0 ? HPACK : D * D) + (kk * 16 + n) * 4;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if (which == 0) {
                    if (j >= a0) store_nt(dst + packed_blk<NT>(a0, j), acc[j]);
                } else {
                    // block (a0, j) of the slab's matrix in accumulator order = block (j, a0)
                    // of its transpose in operand order
                    store_nt(dst + (j * NT + a0) * 256, acc[j]);
                }
            }
        }

        // ---- S <- Gamma_c S + U,  U = sum_i w_i k_i b_i^T  (b = k for H, v for G^T) ----
        // U is a fresh MFMA chain (started from zero, only read afterwards);
        // the decayed running state is combined with it on the VALU.
        f32x4 U[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) U[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
            // 32 tokens per MFMA: lane group kk's eight k-slots e are tokens
            // 32 g2 + 16 (e / 4) + 4 kk + e % 4, i.e. the token pairs
            // p = 16 g2 + 8 h + 2 kk + {0, 1} for h = 0, 1 (a chunk of 16
            // tokens leaves h = 1 empty).
            const uint32_t* tA = reinterpret_cast<const uint32_t*>(sArows);
            const uint32_t* tB = reinterpret_cast<const uint32_t*>(sBcols);
#pragma unroll
            for (int g2 = 0; g2 < (C + 31) / 32; ++g2) {
                constexpr int NH = C >= 32 ? 2 : 1;
                uint32_t ah[4], am[4], al[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) ah[q] = am[q] = al[q] = 0u;
#pragma unroll
                for (int h = 0; h < NH; ++h) {
                    const int p0 = 16 * g2 + 8 * h + 2 * kk;
                    const f32x4 wv = *reinterpret_cast<const f32x4*>(&sW[2 * p0]);
#pragma unroll
                    for (int d = 0; d < 2; ++d) {
                        const uint32_t pr = tA[(p0 + d) * PP + m0 + n];
                        uint32_t hb[2], mb[2], lb[2];
#pragma unroll
                        for (int t = 0; t < 2; ++t) {
                            const float a = __uint_as_float(t ? (pr & 0xffff0000u) : (pr << 16));
                            const float x = a * wv[2 * d + t];
                            // exact split: x = hi + mid + lo, each a bf16
                            hb[t] = __float_as_uint(x) & 0xffff0000u;
                            const float r1 = x - __uint_as_float(hb[t]);
                            mb[t] = __float_as_uint(r1) & 0xffff0000u;
                            lb[t] = __float_as_uint(r1 - __uint_as_float(mb[t])) & 0xffff0000u;
                        }
                        const int q = 2 * h + d;
                        ah[q] = (hb[0] >> 16) | hb[1];
                        am[q] = (mb[0] >> 16) | mb[1];
                        al[q] = (lb[0] >> 16) | lb[1];
                    }
                }
                const bf16x8 Ah = as_bf16x8(ah), Am = as_bf16x8(am), Al = as_bf16x8(al);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int h = 0; h < NH; ++h) {
                        const int p0 = 16 * g2 + 8 * h + 2 * kk;
                        b[2 * h] = tB[p0 * PP + 16 * j + n];
                        b[2 * h + 1] = tB[(p0 + 1) * PP + 16 * j + n];
                    }
                    const bf16x8 Bj = as_bf16x8(b);
                    U[j] = mfma_bf16x32(Ah, Bj, U[j]);
                    U[j] = mfma_bf16x32(Am, Bj, U[j]);
                    U[j] = mfma_bf16x32(Al, Bj, U[j]);
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < C / 16; ++g) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int i = 16 * g + 4 * kk + s;
                    const float a = sArows[i * PD + m0 + n] * sW[i];
#pragma unroll
                    for (int j = 0; j < NT; ++j) U[j] = mfma4(a, sBcols[i * PD + 16 * j + n], U[j]);
                }
            }
        }
        const float G = sGam;
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = G * acc[j] + U[j];
        __syncthreads();
    };

#pragma unroll
    for (int sl = 0; sl < RING; ++sl)
        if (sl < n_chunks) prefetch(sl, sl);
    for (int c = 0; c < n_chunks; c += RING) {
#pragma unroll
        for (int sl = 0; sl < RING; ++sl)
            if (c + sl < n_chunks) step(c + sl, sl);
    }

    // ---- final state (after the last token) ----
    if (which == 0 && final_H) {
        float* dst = final_H + (size_t)bh * D * D;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)(m0 + 4 * kk + r) * D + 16 * j + n] = acc[j][r];
    }
    if (which == 1 && final_G && g_transposed) {
        float* dst = final_G + (size_t)bh * D * D;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)(m0 + 4 * kk + r) * D + 16 * j + n] = acc[j][r];
    }
    if (which == 1 && final_G && !g_transposed) {
        // acc[j][r] = G[16j + n][m0 + 4kk + r]: four consecutive floats of a row of G
        float* dst = final_G + (size_t)bh * D * D;
#pragma unroll
        for (int j = 0; j < NT; ++j)
            *reinterpret_cast<f32x4*>(dst + (size_t)(16 * j + n) * D + m0 + 4 * kk) = acc[j];
    }
}

template <int D, int C, int NW, typename In>
hipError_t launch_chunk_states_nw(const ChunkStatesArgs& a, hipStream_t s) {
    constexpr int RB = D / (16 * NW);
    // ids: 8 XCD lanes x (heads rounded up to a multiple of 8) / 8 x parts
    const long grid = ((a.BH + 7) / 8) * 8 * 2 * RB;
    hipLaunchKernelGGL((chunk_states_kernel<D, C, NW, In>), dim3((unsigned)grid), dim3(64 * NW), 0, s,
                       (const In*)a.k, (const In*)a.v, a.gamma, a.T, a.n_chunks, a.SH, a.SG,
                       a.final_H, a.final_G, a.write_chunks, a.BH, a.work_counter, a.g_transposed);
    return hipGetLastError();
}

template <int D, int C, typename In>
hipError_t launch_chunk_states_t(const ChunkStatesArgs& a, hipStream_t s) {
    // Four waves (64 state rows) per workgroup.  Eight waves (a whole d = 128
    // state per workgroup) would share the key tile better, but must fit two
    // waves per SIMD in 256 registers, where the compiler's allocation
    // rewrites MFMA accumulator inputs early (see codegen_check).
    return launch_chunk_states_nw<D, C, (D >= 64 ? 4 : D / 16), In>(a, s);
}

template <int D, typename In>
static hipError_t dispatch_c(const ChunkStatesArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_chunk_states_t<D, 16, In>(a, s);
        case 32: return launch_chunk_states_t<D, 32, In>(a, s);
        case 64: return launch_chunk_states_t<D, 64, In>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename In>
static hipError_t dispatch_d(const ChunkStatesArgs& a, hipStream_t s) {
    switch (a.d) {
        case 16: return dispatch_c<16, In>(a, s);
        case 32: return dispatch_c<32, In>(a, s);
        case 64: return dispatch_c<64, In>(a, s);
        case 128: return dispatch_c<128, In>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_chunk_states(const ChunkStatesArgs& a, hipStream_t s) {
    return a.bf16 ? dispatch_d<bf16_t>(a, s) : dispatch_d<float>(a, s);
}

}  // namespace mesa
