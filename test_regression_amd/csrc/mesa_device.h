// mesa_device.h -- device helpers shared by the gfx950 Mesa-layer kernels.
//
// Wave64 only.  MFMA layout used throughout (v_mfma_f32_16x16x4_f32, one
// block of 16x16 outputs per instruction): lane l = 16*kk + n holds
//   A operand : A[m = n][k-slot kk]        (one fp32)
//   B operand : B[k-slot kk][col = n]      (one fp32)
//   C/D       : C[row = 4*kk + r][col = n] for r = 0..3 (four fp32)
// The mapping of the 4 k-slots to actual contraction indices is free as long
// as A and B agree; the kernels use k = 16*g + 4*kk + s for sub-step s of
// group g, so that a lane's four A values are contiguous (one 128-bit LDS
// read feeds four MFMAs).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mesa {

typedef float f32x4 __attribute__((ext_vector_type(4)));

// LDS row pitches (floats), measured on gfx950 for the kernels' patterns:
//  - lds_pitch (row length rounded up to 64, plus 4): conflict-free for
//    32-bit accesses where 16 lanes walk a row and the 4 lane groups take 4
//    consecutive rows (the MFMA operand staging and column reads), and a
//    2-way conflict for 128-bit row reads;
//  - lds_pitch_rows (plus 8): conflict-free for 128-bit reads where 16 lanes
//    take 16 consecutive rows and the 4 lane groups 4 consecutive 16-byte
//    pieces of a row; used for tiles that are only ever read that way.
__host__ __device__ constexpr int lds_pitch(int n) { return ((n + 63) / 64) * 64 + 4; }
__host__ __device__ constexpr int lds_pitch_rows(int n) { return ((n + 63) / 64) * 64 + 8; }

// Chunk states in the forward workspace are stored as 16 x 16 blocks of 256
// floats, 16 bytes per lane of a wave: lane 16q + m holds floats
// 4(16q + m)..4(16q + m) + 3 of a block.  H blocks are in MFMA accumulator
// order (those four floats are rows 4q..4q+3 of column m), G blocks in MFMA
// operand order (columns 4q..4q+3 of row m).
__host__ __device__ constexpr int acc_tile_offset(int row, int col) { return ((row >> 2) * 16 + col) * 4 + (row & 3); }
__host__ __device__ constexpr int opnd_tile_offset(int row, int col) { return ((col >> 2) * 16 + row) * 4 + (col & 3); }

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 MFMA: lane 16g + m supplies row m (A) or column m (B) at
// k-slots 8g..8g+7, element e of its eight in bits 16(e % 2) of word e / 2.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 as_bf16x8(const uint32_t (&w)[4]) {
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    return __builtin_bit_cast(bf16x8, u32x4{w[0], w[1], w[2], w[3]});
}
__device__ __forceinline__ f32x4 mfma_bf16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// bf16 stored as raw 16-bit patterns.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) { return __uint_as_float((uint32_t)x.bits << 16); }

// Load 4 consecutive elements (16-byte aligned for float, 8-byte for bf16).
__device__ __forceinline__ f32x4 load4(const float* p) {
    return *reinterpret_cast<const f32x4*>(p);
}
__device__ __forceinline__ f32x4 load4(const bf16_t* p) {
    uint2 u = *reinterpret_cast<const uint2*>(p);
    f32x4 r;
    r[0] = __uint_as_float(u.x << 16);
    r[1] = __uint_as_float(u.x & 0xffff0000u);
    r[2] = __uint_as_float(u.y << 16);
    r[3] = __uint_as_float(u.y & 0xffff0000u);
    return r;
}

// Streaming (non-temporal) stores for outputs that no later instruction of
// the kernel reads: marked for early eviction from the caches, which lets
// HBM writes stream instead of competing with the kernel's reads for cache.
__device__ __forceinline__ void store_nt(float* p, f32x4 v) {
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
}
__device__ __forceinline__ void store_nt(float* p, float v) { __builtin_nontemporal_store(v, p); }

// Ordinary (write-back) store of a lane's 16-byte piece of an output row, for
// row tiles that one store instruction covers only half of each 128-byte
// line of (lane (n, kk) at row n, floats 16 j + 4 kk .. + 3; the next j
// writes the other half).  Streaming stores let the L2 write such half-filled
// lines out more than once: the write counters read up to 1.35x the bytes.
__device__ __forceinline__ void store_row(float* p, f32x4 v) { *reinterpret_cast<f32x4*>(p) = v; }

// Registers holding 4 prefetched input elements (bf16 stays packed until staged).
template <typename In> struct Raw4;
template <> struct Raw4<float> {
    f32x4 v;
    __device__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
    __device__ void zero() { v = f32x4{0.f, 0.f, 0.f, 0.f}; }
    __device__ f32x4 get() const { return v; }
};
template <> struct Raw4<bf16_t> {
    uint2 v;
    __device__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ void zero() { v = make_uint2(0u, 0u); }
    __device__ uint2 raw() const { return v; }
    __device__ f32x4 get() const {
        return f32x4{__uint_as_float(v.x << 16), __uint_as_float(v.x & 0xffff0000u), __uint_as_float(v.y << 16),
                     __uint_as_float(v.y & 0xffff0000u)};
    }
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 16 lanes of a DPP row (lanes 16*kk .. 16*kk+15), i.e. over the
// MFMA column index n.  Every lane of the row gets the same, bit-identical
// value (each step adds two commuted operands).
__device__ __forceinline__ float rowsum16(float v) {
    v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp<0x141>(v);   // row_half_mirror
    v += dpp<0x140>(v);   // row_mirror
    return v;
}

// Sum over the 4 lanes n, n+16, n+32, n+48 (the four DPP rows), i.e. over
// the MFMA k-slot group kk.  The two gfx950 lane swaps pair row 0 with 1 and
// 2 with 3, then the lower half with the upper; every lane adds the same two
// operands, so all four get bit-identical sums.
__device__ __forceinline__ float kslot_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Sum over all 64 lanes (butterfly; every lane gets the same value).
__device__ __forceinline__ float wavesum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Orders this wave's earlier LDS accesses before its later ones (the kernels
// pass data between lanes of one wave through LDS without a block barrier).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Within-chunk log decays.  Lane i < len gets l_i = sum_{s<=i} ln(gamma_s) of
// the chunk's tokens (tokens past the sequence end count as gamma = 1).
// Must be called by a whole wave.
__device__ __forceinline__ float chunk_log_decay_of(float gamma_lane, int valid, int lane) {
    float x = (lane < valid) ? __logf(gamma_lane) : 0.0f;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        float t = __shfl_up(x, o, 64);
        if (lane >= o) x += t;
    }
    return x;
}
__device__ __forceinline__ float chunk_log_decay(const float* gamma_chunk, int valid, int lane) {
    return chunk_log_decay_of(lane < valid ? gamma_chunk[lane] : 1.0f, valid, lane);
}

}  // namespace mesa
