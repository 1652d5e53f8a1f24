// chunk_states.hip -- chunk-boundary states of the Mesa layer (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section "A Camada
// Mesa", bullet "Paralelizacao": the layer keeps the state variables H_t and
// G_t and solves chunks of the sequence in parallel.  With the forget factors
// zeta_{tt'} = prod_{s=t'+1..t} gamma_s the states obey
//   H_t = gamma_t H_{t-1} + k_t k_t^T,   G_t = gamma_t G_{t-1} + v_t k_t^T.
// Over a chunk c of C tokens with within-chunk log decays l_i (prefix sums of
// ln gamma) this is
//   S_{c+1} = e^{l_end} S_c + sum_{i in c} e^{l_end - l_i} a_i b_i^T,
// with (a, b) = (k, k) for H and (k, v) for G^T, S_0 = 0.  This kernel
// produces S_c for every chunk (the state before the chunk's first token)
// and, optionally, the final state after the last token.
//
// Chunk states in the workspace: G as all its 16 x 16 blocks, H (symmetric)
// as the upper triangle of them -- the part the CG kernel reads -- each in
// row-major block order, so a wave stores a block as one 16-byte piece per
// lane (1 KiB contiguous).  An H block is kept in MFMA accumulator order
// (lane 16q + m holds rows 4q..4q+3 of column m); a G block in MFMA operand
// order (lane 16q + m holds columns 4q..4q+3 of row m), which is the A
// operand the CG kernel's output product takes straight from memory.  For
// the backward's adjoint solve (g_transposed) the blocks of G^T are stored
// in operand order instead, the A operand of its G^T g product.  The
// exported final states are full and row-major ([d_v][d_k] for G).
//
// Work split.  A wave owns a fixed list of 16 x 16 output tiles of one state
// and keeps them in MFMA accumulator registers while it walks the chunks in
// order; per chunk a tile gains one (16 x C) x (C x 16) product over the
// chunk's tokens, with the weighted rows w_i a_i as the A operand.
//   - H: only the upper block triangle is formed.  Wave w of an H workgroup
//     takes the tiles of row blocks w and NT-1-w right of the diagonal: NT+1
//     tiles, the same for every wave.  The exported final H gets its lower
//     triangle by mirroring.
//   - G^T (or G with g_transposed): wave w takes row block w of its
//     workgroup's rows and NT/CS column tiles.
// With CS = 2 (few heads of d = 128) the columns are split over two
// workgroups, so a wave holds half as many tiles and twice as many waves run.
// The workgroup stages the chunk's rows and columns it needs in LDS (two
// buffers, one barrier per chunk); the global loads of chunk c + 3 are issued
// while chunk c is multiplied, from clamped addresses so that every wave
// issues the same loads and the compiler can count them, and the states are
// stored without being waited for.
//
// Products: fp32 keys and values on v_mfma_f32_16x16x4_f32.  For bf16 the
// values a_i, b_i are exact bf16, and each weighted value w_i a_i (a float)
// is split exactly into three bf16 parts (the top 8, next 8 and last 8 bits
// of its significand), so three v_mfma_f32_16x16x32_bf16 products sum to the
// float product terms up to the accumulation order.  bf16 tiles are staged
// with two consecutive tokens per 32-bit LDS word (each thread packs a token
// pair of four features into one 16-byte write), so a lane's eight-token
// MFMA operand is four word reads.  Workgroup ids are mapped so that the
// workgroups of one head land on the same XCD (ids congruent mod 8) and
// share its L2 for the key and value tiles.
#include <type_traits>

#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

// Offset (floats) of block (a, b), a <= b, in the packed upper block triangle
// of a d x d state (16 x 16 blocks stored row-major one after another).
template <int NT>
__device__ __forceinline__ int packed_blk(int a, int b) {
    return (a * NT - a * (a - 1) / 2 + (b - a)) * 256;
}

// Inclusive prefix sum over the 64 lanes of a wave: in-row steps on
// row_shr 1, 2, 4, 8, then the row totals carried on by row_bcast 15 (into
// rows 1 and 3) and row_bcast 31 (into rows 2 and 3).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_moved(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_inclusive_sum(float x) {
    x += dpp_moved<0x111, 0xf>(x);
    x += dpp_moved<0x112, 0xf>(x);
    x += dpp_moved<0x114, 0xf>(x);
    x += dpp_moved<0x118, 0xf>(x);
    x += dpp_moved<0x142, 0xa>(x);
    x += dpp_moved<0x143, 0xc>(x);
    return x;
}

// One staged LDS region of F consecutive features of a chunk.
//   bf16: row p holds token pair (2p, 2p + 1); word (p, f) = feature f of
//         token 2p (low half) and 2p + 1 (high half).  The pitch F + 8 puts
//         the four lane groups' rows (2 pairs apart) 16 banks apart.
//   fp32: feature-major, row f holds feature f of the C tokens, so that a
//         lane's four consecutive tokens are one 16-byte read.  The pitch
//         (C rounded up to 64, plus 8) is the one a probe of gfx950's LDS
//         measured free of bank conflicts for 16-byte reads where 16 lanes
//         take 16 consecutive rows (a pitch of 64 + 4 lost 17% of the cycles).
template <int F, int C, bool BF>
struct StageTile {
    static constexpr int FG = F / 4;                        // 4-feature groups of a token
    static constexpr int PITCH = BF ? F + 8 : (C + 63) / 64 * 64 + 8;   // 32-bit words per LDS row
    static constexpr int WORDS = (BF ? C / 2 : F) * PITCH;
    // bf16: a token pair x 4 features; fp32: 4 tokens x 4 features
    static constexpr int UNITS = (BF ? C / 2 : C / 4) * FG;
};

template <int D, int C, int NW, int CS, bool BF>
struct K1Shape {
    static constexpr int NT = D / 16;          // 16 x 16 tiles per state row block
    static constexpr int RB = D / (16 * NW);   // row blocks of NW tiles per G^T state
    static constexpr int NTW = NT / CS;        // column tiles per G wave
    static constexpr int PAIRS = (NT + 1) / 2; // H waves (row blocks w and NT-1-w)
    static constexpr int HTILES = NT == 1 ? 1 : NT + 1;
    static constexpr int HPARTS = CS;          // H workgroups per head
    static constexpr int GPARTS = RB * CS;     // G workgroups per head
    static constexpr int PARTS = HPARTS + GPARTS;
    // H tiles per wave in H part h (CS = 2: the NT+1 tiles split 5 / 4)
    static constexpr int HT0 = CS == 1 ? HTILES : (HTILES + 1) / 2;
    static constexpr int HT1 = HTILES - HT0;
    using KT = StageTile<D, C, BF>;            // H: the whole key tile
    using AT = StageTile<16 * NW, C, BF>;      // G: the workgroup's rows
    using BT = StageTile<D / CS, C, BF>;       // G: the workgroup's columns
    static constexpr int HBUF = KT::WORDS + C + 4;
    static constexpr int GBUF = AT::WORDS + BT::WORDS + C + 4;
    static constexpr int BUF = HBUF > GBUF ? HBUF : GBUF;   // words per LDS buffer
};

// Raw buffer resource over `bytes` bytes from `base`: loads past the end
// return zeros and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t k1_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Per-thread offsets of one staged region's units: the byte offset of the
// unit within a chunk's rows of the input and its LDS word offset.  Unit
// indices past the region are clamped onto its last unit, whose LDS write
// then repeats with the same data.
//   bf16: a token pair x 4 features, 4-feature groups fastest (a wave reads
//         whole pair rows): two 8-byte loads, one 16-byte LDS write.
//   fp32: 4 tokens x 4 features (four 16-byte loads, one per token), with
//         eight token quads fastest, so that a wave reads 128-byte pieces of
//         8 rows and its four 16-byte LDS writes (one per feature row, four
//         tokens each) go to eight distinct 16-byte slots per lane octet.
template <typename Tl, int NTHR, int D, int ES>
struct UnitOffsets {
    static constexpr int U = (Tl::UNITS + NTHR - 1) / NTHR;
    int g[U], l[U];
    __device__ __forceinline__ UnitOffsets(int f0, int tid) {
#pragma unroll
        for (int e = 0; e < U; ++e) {
            const int u = min(tid + e * NTHR, Tl::UNITS - 1);
            if constexpr (ES == 2) {
                const int row = u / Tl::FG, fg = u % Tl::FG;
                g[e] = (2 * row * D + f0 + 4 * fg) * ES;
                l[e] = row * Tl::PITCH + 4 * fg;
            } else {
                constexpr int TQ = Tl::UNITS / Tl::FG;           // token quads
                constexpr int QL = TQ < 8 ? TQ : 8;
                const int tq = (u / (QL * Tl::FG)) * QL + u % QL, fg = (u / QL) % Tl::FG;
                g[e] = (4 * tq * D + f0 + 4 * fg) * ES;
                l[e] = 4 * fg * Tl::PITCH + 4 * tq;
            }
        }
    }
};

template <typename Tl, int NTHR, int D, typename In, typename Ld>
__device__ __forceinline__ void k1_load(Ld (&r)[(Tl::UNITS + NTHR - 1) / NTHR][sizeof(In) == 2 ? 2 : 4],
                                        __amdgpu_buffer_rsrc_t rs, const UnitOffsets<Tl, NTHR, D, sizeof(In)>& o) {
    constexpr int U = (Tl::UNITS + NTHR - 1) / NTHR;
#pragma unroll
    for (int e = 0; e < U; ++e) {
        if constexpr (sizeof(In) == 2) {
            r[e][0] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, o.g[e], 0, 0));
            r[e][1] = __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(rs, o.g[e] + 2 * D, 0, 0));
        } else {
#pragma unroll
            for (int q = 0; q < 4; ++q)
                r[e][q] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, o.g[e] + q * 4 * D, 0, 0));
        }
    }
}

// Write the loaded units into LDS (rows past the sequence arrived as zeros).
template <typename Tl, int NTHR, int D, typename In, typename Ld>
__device__ __forceinline__ void k1_stage(const Ld (&r)[(Tl::UNITS + NTHR - 1) / NTHR][sizeof(In) == 2 ? 2 : 4],
                                         float* dst, const UnitOffsets<Tl, NTHR, D, sizeof(In)>& o) {
    constexpr int U = (Tl::UNITS + NTHR - 1) / NTHR;
#pragma unroll
    for (int e = 0; e < U; ++e) {
        if constexpr (sizeof(In) == 2) {
            const uint2 x = r[e][0], y = r[e][1];
            // word f = (feature f of token 2p) | (feature f of token 2p + 1) << 16
            typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
            const u32x4v wd{(x.x & 0xffffu) | (y.x << 16), (x.x >> 16) | (y.x & 0xffff0000u),
                            (x.y & 0xffffu) | (y.y << 16), (x.y >> 16) | (y.y & 0xffff0000u)};
            *reinterpret_cast<u32x4v*>(dst + o.l[e]) = wd;
        } else {
            // feature row 4 fg + j gets tokens 4 tq .. 4 tq + 3
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<f32x4*>(dst + o.l[e] + j * Tl::PITCH) =
                    f32x4{r[e][0][j], r[e][1][j], r[e][2][j], r[e][3][j]};
        }
    }
}

// The per-wave chunk walk.  KIND 0: H tiles (TW tiles starting at tile T0
// of the list of row-block pair pr); KIND 1: G^T (or G) tiles (row block
// grow, column tiles gcol0 ..).  WRITE: store the chunk states.
// MODE 0: the workgroup stages only the rows and columns of its own kind
// (H: the key tile; G: fA.. of the row source, fB.. of the column source).
// MODE 1: the workgroup stages the whole key and value tiles and mixes H and
// G waves (fA = fB = 0).
template <int D, int C, int NW, int CS, typename In, int KIND, int TW, int T0, bool WRITE, int MODE>
__device__ __forceinline__ void chunk_states_walk(const In* __restrict__ k, const In* __restrict__ v,
                                                  const float* __restrict__ gamma, int T, int n_chunks,
                                                  float* __restrict__ Sout, float* __restrict__ final_S,
                                                  int g_transposed, long bh, int pr, int grow, int gcol0, int fA,
                                                  int fB, float* lds) {
    constexpr bool BF = sizeof(In) == 2;
    using S = K1Shape<D, C, NW, CS, BF>;
    constexpr int NT = S::NT;
    constexpr int NTHR = 64 * NW;
    constexpr int HPACK = D * (D + 16) / 2;    // floats of a packed upper block triangle
    using Ld = std::conditional_t<BF, uint2, f32x4>;
    constexpr int NL = BF ? 2 : 4;
    // staged regions: MODE 0 H one key region (rows and columns), G a row
    // region and a column region; MODE 1 the key region, then the value region
    using TA = std::conditional_t<KIND == 0 || MODE == 1, typename S::KT, typename S::AT>;
    using TB = std::conditional_t<KIND == 0 || MODE == 1, typename S::KT, typename S::BT>;
    constexpr bool LOADA = MODE == 1 || KIND == 1;
    constexpr int UA = LOADA ? (TA::UNITS + NTHR - 1) / NTHR : 1;
    constexpr int UB = (TB::UNITS + NTHR - 1) / NTHR;
    constexpr int BUF = MODE == 1 ? 2 * S::KT::WORDS + C + 4 : S::BUF;
    constexpr int WOFF = MODE == 1 ? 2 * S::KT::WORDS : (KIND == 0 ? 0 : TA::WORDS) + TB::WORDS;
    constexpr int NR = KIND == 0 && NT > 1 ? 2 : 1;   // row blocks a wave's tiles come from
    const bool gt = KIND == 1 && g_transposed;
    // region offsets of the A and B operands (MODE 1: key region 0, value region 1)
    const int AOFF = MODE == 1 ? (gt ? S::KT::WORDS : 0) : 0;
    const int BOFF = MODE == 1 ? (KIND == 0 || gt ? 0 : S::KT::WORDS) : (KIND == 0 ? 0 : TA::WORDS);

    typedef uint32_t u32x4s __attribute__((ext_vector_type(4)));
    const int tid0 = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int lane = tid0 & 63;
    const int n = lane & 15, kk = lane >> 4;

    // this wave's tiles: row blocks r0 (tiles t' < split) and r1, column of tile t' = T0 + t
    const bool active = KIND == 1 || MODE == 1 || S::PAIRS == NW || w < S::PAIRS;
    const int r0 = KIND == 0 ? pr : grow;
    const int r1 = KIND == 0 ? NT - 1 - pr : grow;
    const int split = KIND == 0 ? NT - pr : TW + T0;
    auto tile_first = [&](int t) { return T0 + t < split; };
    auto tile_col = [&](int t) {
        if constexpr (KIND == 0) return T0 + t < split ? pr + T0 + t : T0 + t - 1;
        else return gcol0 + t;
    };
    // A operand feature offset of row block r in its region; B operand of tile t
    auto a_off = [&](int r) { return 16 * r - fA; };
    auto b_off = [&](int t) { return 16 * tile_col(t) - fB; };

    constexpr int ES = sizeof(In);
    // MODE 1: A loads the keys and B the values; MODE 0: each its operand's source
    const In* srcA = (MODE == 1 ? k : gt ? v : k) + (size_t)bh * T * D;
    const In* srcB = (MODE == 1 ? v : KIND == 0 || gt ? k : v) + (size_t)bh * T * D;
    const float* gh = gamma + (size_t)bh * T;
    const UnitOffsets<TA, NTHR, D, ES> oA(fA, tid0);
    const UnitOffsets<TB, NTHR, D, ES> oB(fB, tid0);

    f32x4 acc[TW];
#pragma unroll
    for (int t = 0; t < TW; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    Ld ra[2][UA][NL], rbv[2][UB][NL];
    float greg[2];
    auto load = [&](int c, int sl) {
        // the chunk's rows as a buffer: rows past the sequence read as zeros
        const int t0 = min(c, n_chunks - 1) * C;
        const int rows = min(C, T - t0);
        if constexpr (LOADA) k1_load<TA, NTHR, D, In>(ra[sl], k1_rsrc(srcA + (size_t)t0 * D, rows * D * ES), oA);
        k1_load<TB, NTHR, D, In>(rbv[sl], k1_rsrc(srcB + (size_t)t0 * D, rows * D * ES), oB);
        greg[sl] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(k1_rsrc(gh + t0, rows * 4),
                                                                                  (tid0 & 63) * 4, 0, 0));
    };
    auto stage = [&](int c, int sl, int buf) {
        float* base = lds + buf * BUF;
        const int valid = min(C, T - c * C);
        // MODE 1: keys into region 0, values into region 1
        if constexpr (LOADA) k1_stage<TA, NTHR, D, In>(ra[sl], base + (MODE == 1 ? 0 : AOFF), oA);
        k1_stage<TB, NTHR, D, In>(rbv[sl], base + (MODE == 1 ? S::KT::WORDS : BOFF), oB);
        // within-chunk log decays (tokens past the end count as gamma = 1):
        // an inclusive scan over the wave on DPP moves, computed by every
        // wave (no branch around it) and written by wave 0
        const float l = wave_inclusive_sum(lane < valid ? __logf(greg[sl]) : 0.f);
        const float lend = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l), C - 1));
        if (w == 0) {
            if (lane < C) base[WOFF + lane] = __expf(lend - l);
            if (lane == 0) base[WOFF + C] = __expf(lend);
        }
    };
    auto store_states = [&](int c) {
        // one 16-byte piece per lane per 16 x 16 block (non-temporal for fp32
        // inputs; plain write-back stores measured faster with bf16 inputs)
        constexpr int SB = (KIND == 0 ? HPACK : D * D) * 4;
        const __amdgpu_buffer_rsrc_t rs = k1_rsrc(Sout + (size_t)c * (SB / 4), SB);
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int row = tile_first(t) ? r0 : r1, col = tile_col(t);
            // G: block (row, col) of the slab's matrix in accumulator order =
            // block (col, row) of its transpose in operand order
            const int blk = KIND == 0 ? packed_blk<NT>(row, col) : (col * NT + row) * 256;
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4s, acc[t]), rs, lane * 16, blk * 4, BF ? 0 : 2);
        }
    };
    auto multiply = [&](int buf) {
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int ln = tid & 63, nn = ln & 15, kq = ln >> 4;
        const float* base = lds + buf * BUF;
        const float* sA = base + AOFF;
        const float* sB = base + BOFF;
        const float* sW = base + WOFF;
        // U is a fresh MFMA chain per tile (started from zero, only read
        // afterwards); the decayed running state is combined with it on the VALU.
        f32x4 U[TW];
#pragma unroll
        for (int t = 0; t < TW; ++t) U[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
            // 32 tokens per MFMA: lane group kq's eight k-slots e are tokens
            // 32 g2 + 16 (e / 4) + 4 kq + e % 4, i.e. the token pairs
            // p = 16 g2 + 8 h + 2 kq + {0, 1} for h = 0, 1 (a chunk of 16
            // tokens leaves h = 1 empty).
            const uint32_t* tA = reinterpret_cast<const uint32_t*>(sA);
            const uint32_t* tB = reinterpret_cast<const uint32_t*>(sB);
            constexpr int NH = C >= 32 ? 2 : 1;
#pragma unroll
            for (int g2 = 0; g2 < (C + 31) / 32; ++g2) {
                bf16x8 Ah[NR], Am[NR], Al[NR];
#pragma unroll
                for (int ri = 0; ri < NR; ++ri) {
                    const int aoff = a_off(ri == 0 ? r0 : r1);
                    uint32_t ah[4], am[4], al[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) ah[q] = am[q] = al[q] = 0u;
#pragma unroll
                    for (int h = 0; h < NH; ++h) {
                        const int p0 = 16 * g2 + 8 * h + 2 * kq;
                        const f32x4 wv = *reinterpret_cast<const f32x4*>(&sW[2 * p0]);
#pragma unroll
                        for (int d = 0; d < 2; ++d) {
                            const uint32_t pr = tA[(p0 + d) * TA::PITCH + aoff + nn];
                            uint32_t hb[2], mb[2], lb[2];
#pragma unroll
                            for (int s = 0; s < 2; ++s) {
                                const float a = __uint_as_float(s ? (pr & 0xffff0000u) : (pr << 16));
                                const float x = a * wv[2 * d + s];
                                // exact split: x = hi + mid + lo, each a bf16
                                hb[s] = __float_as_uint(x) & 0xffff0000u;
                                const float r1f = x - __uint_as_float(hb[s]);
                                mb[s] = __float_as_uint(r1f) & 0xffff0000u;
                                lb[s] = __float_as_uint(r1f - __uint_as_float(mb[s])) & 0xffff0000u;
                            }
                            const int q = 2 * h + d;
                            ah[q] = (hb[0] >> 16) | hb[1];
                            am[q] = (mb[0] >> 16) | mb[1];
                            al[q] = (lb[0] >> 16) | lb[1];
                        }
                    }
                    Ah[ri] = as_bf16x8(ah);
                    Am[ri] = as_bf16x8(am);
                    Al[ri] = as_bf16x8(al);
                }
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const int boff = b_off(t);
                    uint32_t b[4] = {0u, 0u, 0u, 0u};
#pragma unroll
                    for (int h = 0; h < NH; ++h) {
                        const int p0 = 16 * g2 + 8 * h + 2 * kq;
                        b[2 * h] = tB[p0 * TB::PITCH + boff + nn];
                        b[2 * h + 1] = tB[(p0 + 1) * TB::PITCH + boff + nn];
                    }
                    const bf16x8 Bj = as_bf16x8(b);
                    const bool f = NR == 1 || tile_first(t);
                    U[t] = mfma_bf16x32(f ? Ah[0] : Ah[NR - 1], Bj, U[t]);
                    U[t] = mfma_bf16x32(f ? Am[0] : Am[NR - 1], Bj, U[t]);
                    U[t] = mfma_bf16x32(f ? Al[0] : Al[NR - 1], Bj, U[t]);
                }
            }
        } else {
            // MFMA (g, s) contracts over tokens 16 g + 4 kq + s (kq = 0..3):
            // a lane's operands for s = 0..3 are four consecutive tokens of
            // one feature row, one 16-byte read each.
#pragma unroll
            for (int g = 0; g < C / 16; ++g) {
                const int i0 = 16 * g + 4 * kq;
                const f32x4 wv = *reinterpret_cast<const f32x4*>(&sW[i0]);
                f32x4 a[NR];
#pragma unroll
                for (int ri = 0; ri < NR; ++ri)
                    a[ri] = *reinterpret_cast<const f32x4*>(&sA[(a_off(ri == 0 ? r0 : r1) + nn) * TA::PITCH + i0]) * wv;
#pragma unroll
                for (int t = 0; t < TW; ++t) {
                    const bool f = NR == 1 || tile_first(t);
                    const f32x4 b = *reinterpret_cast<const f32x4*>(&sB[(b_off(t) + nn) * TB::PITCH + i0]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) U[t] = mfma4(f ? a[0][s] : a[NR - 1][s], b[s], U[t]);
                }
            }
        }
        const float G = sW[C];
#pragma unroll
        for (int t = 0; t < TW; ++t) acc[t] = G * acc[t] + U[t];
    };

    // Pipeline, one barrier per chunk: chunk c is multiplied from buffer
    // c & 1, then chunk c + 1 (loaded two steps earlier into register slot
    // (c+1) & 1) is staged into the other buffer -- its vector work and LDS
    // writes can run under the tail of the MFMA chain -- and chunk c + 3's
    // loads go into the freed slot.  At the last chunk the staging repeats
    // chunk n - 1 into a buffer no wave reads any more.
    load(0, 0);
    load(1, 1);
    stage(0, 0, 0);
    load(2, 0);
    __syncthreads();
    auto step = [&](int c, int sl, int buf) {
        if (active) {
            if constexpr (WRITE) store_states(c);
            multiply(buf);
        }
        stage(c + 1, sl, buf ^ 1);
        load(c + 3, sl);
        __syncthreads();
    };
    for (int c = 0; c < n_chunks; c += 2) {
        step(c, 1, 0);
        if (c + 1 < n_chunks) step(c + 1, 0, 1);
    }

    // ---- final state (after the last token) ----
    if (final_S && active) {
        float* dst = final_S + (size_t)bh * D * D;
#pragma unroll
        for (int t = 0; t < TW; ++t) {
            const int row = tile_first(t) ? r0 : r1, col = tile_col(t);
            if (KIND == 0 || gt) {
                // acc[t][q] = S[16 row + 4 kk + q][16 col + n]
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[(size_t)(16 * row + 4 * kk + q) * D + 16 * col + n] = acc[t][q];
                // H's lower triangle by symmetry
                if (KIND == 0 && col != row)
                    *reinterpret_cast<f32x4*>(dst + (size_t)(16 * col + n) * D + 16 * row + 4 * kk) = acc[t];
            } else {
                // acc[t][q] = G[16 col + n][16 row + 4 kk + q]: four consecutive floats of a row of G
                *reinterpret_cast<f32x4*>(dst + (size_t)(16 * col + n) * D + 16 * row + 4 * kk) = acc[t];
            }
        }
    }
}

// NW: waves per workgroup.  CS: column splits of a G state (1 or 2).
template <int D, int C, int NW, int CS, typename In, bool WRITE>
__global__ __launch_bounds__(64 * NW) void chunk_states_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma, int T, int n_chunks,
    float* __restrict__ SH, float* __restrict__ SG, float* __restrict__ final_H, float* __restrict__ final_G,
    long BH, int* __restrict__ work_counter, int g_transposed) {
    using S = K1Shape<D, C, NW, CS, sizeof(In) == 2>;
    __shared__ alignas(16) float lds[2 * S::BUF];
    // the chunk-claim counter of the CG/output kernel that runs next
    if (work_counter && blockIdx.x == 0 && threadIdx.x == 0) *work_counter = 0;

    // XCD-aware id: consecutive ids go round-robin over the 8 XCDs, so the
    // PARTS workgroups of head bh get ids xcd + 8*(slot) with equal xcd.
    const long xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const long bh = (slot / S::PARTS) * 8 + xcd;
    const int part = (int)(slot % S::PARTS);
    if (bh >= BH) return;                      // whole workgroup: no barrier is skipped
    constexpr int HPACK = D * (D + 16) / 2;
    float* SHh = WRITE ? SH + (size_t)bh * n_chunks * HPACK : nullptr;
    float* SGh = WRITE ? SG + (size_t)bh * n_chunks * D * D : nullptr;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (part < S::HPARTS) {
        // wave w: row-block pair (w, NT-1-w)
        if (part == 0)
            chunk_states_walk<D, C, NW, CS, In, 0, S::HT0, 0, WRITE, 0>(k, v, gamma, T, n_chunks, SHh, final_H, 0,
                                                                        bh, w, 0, 0, 0, 0, lds);
        else if constexpr (S::HT1 > 0)
            chunk_states_walk<D, C, NW, CS, In, 0, S::HT1, S::HT0, WRITE, 0>(k, v, gamma, T, n_chunks, SHh,
                                                                             final_H, 0, bh, w, 0, 0, 0, 0, lds);
    } else {
        // row block rb * NW + w, column tiles cs * NTW ..
        const int g = part - S::HPARTS, rb = g / CS, cs = g % CS;
        chunk_states_walk<D, C, NW, CS, In, 1, S::NTW, 0, WRITE, 0>(
            k, v, gamma, T, n_chunks, SGh, final_G, g_transposed, bh, 0, rb * NW + w, cs * S::NTW, rb * 16 * NW,
            cs * (D / CS), lds);
    }
}

// d = 128 with fp32 keys and values: four workgroups of eight waves per
// head, each staging the whole key and value tiles (the fp32 products run
// at the fp32 MFMA rate, so the work is spread evenly over the SIMDs: one
// workgroup per CU, two waves per SIMD).  Workgroup q takes row-block pair
// (q, 7-q) of H, its nine tiles split 3/2/2/2 over waves 0-3, and row blocks
// 2q, 2q+1 of G^T in halves of four column tiles on waves 4-7, so that the
// two waves of a SIMD (w and w+4) hold six or seven tiles.
template <int C, typename In, bool WRITE>
__global__ __launch_bounds__(512) void chunk_states_full_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma, int T, int n_chunks,
    float* __restrict__ SH, float* __restrict__ SG, float* __restrict__ final_H, float* __restrict__ final_G,
    long BH, int* __restrict__ work_counter, int g_transposed) {
    constexpr int D = 128;
    using S = K1Shape<D, C, 8, 1, sizeof(In) == 2>;
    __shared__ alignas(16) float lds[2 * (2 * S::KT::WORDS + C + 4)];
    if (work_counter && blockIdx.x == 0 && threadIdx.x == 0) *work_counter = 0;
    // An (empty) accumulator-register clobber: it makes the compiler keep the
    // MFMA accumulators in AGPRs.  Without it this 512-thread kernel gets the
    // all-VGPR MFMA form, where accumulator inputs are rewritten a few wait
    // states after issue (the pattern codegen_check rejects).
    asm volatile("" ::: "a0");
    // the 4 workgroups of head bh on one XCD
    const long xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const long bh = (slot / 4) * 8 + xcd;
    const int q = (int)(slot % 4);
    if (bh >= BH) return;
    constexpr int HPACK = D * (D + 16) / 2;
    float* SHh = WRITE ? SH + (size_t)bh * n_chunks * HPACK : nullptr;
    float* SGh = WRITE ? SG + (size_t)bh * n_chunks * D * D : nullptr;
    const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
#define K1_H(TW, T0)                                                                                            \
    chunk_states_walk<D, C, 8, 1, In, 0, TW, T0, WRITE, 1>(k, v, gamma, T, n_chunks, SHh, final_H, 0, bh, q, 0, 0, \
                                                            0, 0, lds)
    switch (w) {
        case 0: K1_H(3, 0); break;
        case 1: K1_H(2, 3); break;
        case 2: K1_H(2, 5); break;
        case 3: K1_H(2, 7); break;
        default:
            chunk_states_walk<D, C, 8, 1, In, 1, 4, 0, WRITE, 1>(k, v, gamma, T, n_chunks, SGh, final_G,
                                                                 g_transposed, bh, 0, 2 * q + ((w - 4) >> 1),
                                                                 ((w - 4) & 1) * 4, 0, 0, lds);
    }
#undef K1_H
}

template <int D, int C, int NW, int CS, typename In>
hipError_t launch_chunk_states_nw(const ChunkStatesArgs& a, hipStream_t s) {
    using S = K1Shape<D, C, NW, CS, sizeof(In) == 2>;
    // ids: 8 XCD lanes x (heads rounded up to a multiple of 8) / 8 x parts
    const long grid = ((a.BH + 7) / 8) * 8 * S::PARTS;
    if (a.write_chunks)
        hipLaunchKernelGGL((chunk_states_kernel<D, C, NW, CS, In, true>), dim3((unsigned)grid), dim3(64 * NW), 0, s,
                           (const In*)a.k, (const In*)a.v, a.gamma, a.T, a.n_chunks, a.SH, a.SG, a.final_H,
                           a.final_G, a.BH, a.work_counter, a.g_transposed);
    else
        hipLaunchKernelGGL((chunk_states_kernel<D, C, NW, CS, In, false>), dim3((unsigned)grid), dim3(64 * NW), 0,
                           s, (const In*)a.k, (const In*)a.v, a.gamma, a.T, a.n_chunks, a.SH, a.SG, a.final_H,
                           a.final_G, a.BH, a.work_counter, a.g_transposed);
    return hipGetLastError();
}

template <int D, int C, typename In>
hipError_t launch_chunk_states_t(const ChunkStatesArgs& a, hipStream_t s) {
    // Four waves (64 state rows) per workgroup at d >= 64.  At d = 128 the
    // columns are split in two for fp32 inputs (whose unsplit G workgroup
    // would need 103 KB of LDS, one workgroup per CU) and when whole column
    // sets would leave fewer than two workgroups per CU.
    constexpr int NW = D >= 64 ? 4 : D / 16;
    if constexpr (D == 128 && sizeof(In) == 4) {
        const long grid = ((a.BH + 7) / 8) * 8 * 4;
        if (a.write_chunks)
            hipLaunchKernelGGL((chunk_states_full_kernel<C, In, true>), dim3((unsigned)grid), dim3(512), 0, s,
                               (const In*)a.k, (const In*)a.v, a.gamma, a.T, a.n_chunks, a.SH, a.SG, a.final_H,
                               a.final_G, a.BH, a.work_counter, a.g_transposed);
        else
            hipLaunchKernelGGL((chunk_states_full_kernel<C, In, false>), dim3((unsigned)grid), dim3(512), 0, s,
                               (const In*)a.k, (const In*)a.v, a.gamma, a.T, a.n_chunks, a.SH, a.SG, a.final_H,
                               a.final_G, a.BH, a.work_counter, a.g_transposed);
        return hipGetLastError();
    } else {
        if constexpr (D == 128)
            if (a.BH * K1Shape<D, C, NW, 1, true>::PARTS < 512) return launch_chunk_states_nw<D, C, NW, 2, In>(a, s);
        return launch_chunk_states_nw<D, C, NW, 1, In>(a, s);
    }
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
