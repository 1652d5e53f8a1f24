// hawk.hip -- the recurrence of the Hawk layer of the Hawk-Mesa hybrid (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section
// "Arquitetura (MesaNet)", bullet "Variante Hibrida": the hybrid model
// alternates LRU (Hawk) layers with Mesa layers.  The page names the layer
// only; the recurrence here is Hawk's published real-gated linear recurrent
// unit, per channel d with gate pre-activations ga, gx:
//   r_t = sigmoid(ga_t),  i_t = sigmoid(gx_t),  log a_t = -c softplus(-lam_d) r_t
//   h_t = a_t h_{t-1} + sqrt(1 - a_t^2) i_t x_t
// (1 - a^2 = 1 - e^{2 log a} is evaluated without cancellation for a near 1).
//
// It is HBM-bound and sequential in t.  Two schedules:
//  - one pass (wide shapes: many 64-channel blocks).  A workgroup of 8
//    waves owns 64 consecutive channels of one sequence for all T, one
//    channel per lane.  The tokens go by in rounds of 8 x 8: wave w takes
//    tokens 8w..8w+7 of the round, forms their gates and the segment's prefix
//    decay products and states from zero, and publishes the segment's
//    (product, end state) in LDS; after one barrier every wave folds the
//    earlier segments into its start state, writes its eight outputs as
//    independent FMAs, and carries the round's end state on.  The next
//    round's rows are in flight while a round computes, so each input is
//    read once from HBM and each gate is formed once;
//  - two passes (few channel blocks and long sequences, where one workgroup
//    per block would leave the GPU idle): pass 1 reduces each (sequence,
//    chunk, channel) to its decay product P_c and its end state s_c from
//    zero; pass 2 folds the earlier chunks' (P, s) into the chunk's start
//    state and rescans the chunk, writing h.  A thread owns four consecutive
//    channels (one 8- or 16-byte piece per row; one channel when rows or
//    pointers are not aligned for that) of one chunk; consecutive threads
//    take consecutive channels, so every load and store of a wave is one
//    contiguous row piece.
#include <type_traits>

#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

constexpr int kHawkUnroll = 8;

__device__ __forceinline__ float hawk_softplus(float z) { return z > 20.f ? z : log1pf(__expf(z)); }
// The gates and the input scale use the hardware reciprocal and square root
// (about 1 ulp each) instead of correctly rounded division and sqrt
// sequences: those made the scan ALU-bound.
__device__ __forceinline__ float hawk_sigmoid(float z) { return __builtin_amdgcn_rcpf(1.0f + __expf(-z)); }

// V consecutive channels of one row, loaded as one 4V- or 2V-byte piece
// (V = 1: a single element).
template <typename In, int V> struct HawkVec;
template <typename In> struct HawkVec<In, 1> {
    In v[1];
    __device__ __forceinline__ void load(const In* p) { v[0] = *p; }
    __device__ __forceinline__ float get(int) const { return to_f32(v[0]); }
};
template <> struct HawkVec<float, 4> {
    f32x4 v;
    __device__ __forceinline__ void load(const float* p) { v = *reinterpret_cast<const f32x4*>(p); }
    __device__ __forceinline__ float get(int i) const { return v[i]; }
};
template <> struct HawkVec<bf16_t, 4> {
    uint2 v;
    __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint2*>(p); }
    __device__ __forceinline__ float get(int i) const {
        const uint32_t w = i < 2 ? v.x : v.y;
        return __uint_as_float((i & 1) ? (w & 0xffff0000u) : (w << 16));
    }
};

template <int V>
__device__ __forceinline__ void store_v(float* p, const float (&x)[V]) {
    if constexpr (V == 4) *reinterpret_cast<f32x4*>(p) = f32x4{x[0], x[1], x[2], x[3]};
    else p[0] = x[0];
}

// One step's decay (as its base-2 log and value) and input term, given the
// channel's scale csp2 = c softplus(-lam) log2(e): log2 a = -csp2 r.
// 1 - a^2 = 1 - 2^{2 log2 a} is the short Taylor series in l = log2 a where
// the subtraction would cancel (2 l ln 2 > -1/16: the first dropped term is
// below 2^-24 relative), and 1 - a*a elsewhere (a < 0.97, so 1 - a*a > 0.06
// keeps ~23 bits).  The input term sqrt(1 - a^2) x / (1 + e^{-gx}) is
// formed with one reciprocal square root, as
// (1 - a^2) x rsq((1 - a^2)(1 + e^{-gx})^2); the floor on the rsq argument
// keeps 1 - a^2 = 0 (a closed gate) at exactly zero.
__device__ __forceinline__ void hawk_step_f(float xv, float gav, float gxv, float csp2, float& log2a, float& a,
                                            float& u) {
    // 1 - 2^{k l} = -sum_n (k l)^n / n!, k = 2 ln 2, to fifth order
    constexpr float k1 = 1.3862943611198906f;     // 2 ln 2
    constexpr float k2 = k1 * k1 / 2.f, k3 = k2 * k1 / 3.f, k4 = k3 * k1 / 4.f, k5 = k4 * k1 / 5.f;
    const float r = hawk_sigmoid(gav);
    const float q = 1.0f + __expf(-gxv);
    log2a = -csp2 * r;
    a = __builtin_amdgcn_exp2f(log2a);
    const float l = log2a;
    const float taylor = -l * (k1 + l * (k2 + l * (k3 + l * (k4 + l * k5))));
    // a lane select, written out: in the scan loops the compiler otherwise
    // turns it into a divergent branch around the series
    const float direct = 1.f - a * a;
    const unsigned long long near1 = __builtin_amdgcn_ballot_w64(l > -0.0625f / k1);
    float oma;
    asm("v_cndmask_b32_e64 %0, %1, %2, %3" : "=v"(oma) : "v"(direct), "v"(taylor), "s"(near1));
    u = xv * oma * __builtin_amdgcn_rsqf(fmaxf(oma * q * q, 1.17549435e-38f));
}

// The channel's decay scale in base-2 units, c softplus(-lam) log2(e).
__device__ __forceinline__ float hawk_scale2(float c, float lam) {
    return c * hawk_softplus(-lam) * 1.4426950408889634f;
}

// A thread owns channels d .. d+V-1 of one chunk of one sequence.
template <typename In, int V>
__global__ __launch_bounds__(256) void hawk_summary_kernel(const In* __restrict__ x, const In* __restrict__ ga,
                                                           const In* __restrict__ gx, const float* __restrict__ lam,
                                                           float c, int T, int D, int nc, long n_threads,
                                                           float* __restrict__ Plog, float* __restrict__ S) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= n_threads) return;
    const int DV = D / V;
    const int d = V * (int)(g % DV);
    const long rem = g / DV;
    const int ch = (int)(rem % nc);
    const long b = rem / nc;
    const int t0 = ch * kHawkChunk, t1 = min(T, t0 + kHawkChunk);
    float csp[V], h[V], lsum[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        csp[q] = hawk_scale2(c, lam[d + q]);
        h[q] = 0.f;
        lsum[q] = 0.f;
    }
    size_t i = ((size_t)b * T + t0) * D + d;
    int t = t0;
    for (; t + kHawkUnroll <= t1; t += kHawkUnroll) {
        HawkVec<In, V> xr[kHawkUnroll], ar[kHawkUnroll], gr[kHawkUnroll];
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            xr[u].load(x + i + (size_t)u * D);
            ar[u].load(ga + i + (size_t)u * D);
            gr[u].load(gx + i + (size_t)u * D);
        }
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u)
#pragma unroll
            for (int q = 0; q < V; ++q) {
                float la, av, vv;
                hawk_step_f(xr[u].get(q), ar[u].get(q), gr[u].get(q), csp[q], la, av, vv);
                h[q] = av * h[q] + vv;
                lsum[q] += la;
            }
        i += (size_t)kHawkUnroll * D;
    }
    for (; t < t1; ++t, i += D) {
        HawkVec<In, V> xr, ar, gr;
        xr.load(x + i);
        ar.load(ga + i);
        gr.load(gx + i);
#pragma unroll
        for (int q = 0; q < V; ++q) {
            float la, av, vv;
            hawk_step_f(xr.get(q), ar.get(q), gr.get(q), csp[q], la, av, vv);
            h[q] = av * h[q] + vv;
            lsum[q] += la;
        }
    }
    const size_t j = ((size_t)b * nc + ch) * D + d;
    store_v<V>(Plog + j, lsum);   // log2 of the chunk's decay product
    store_v<V>(S + j, h);         // the chunk's end state from zero
}

template <typename In, int V>
__global__ __launch_bounds__(256) void hawk_scan_kernel(const In* __restrict__ x, const In* __restrict__ ga,
                                                        const In* __restrict__ gx, const float* __restrict__ lam,
                                                        float c, const float* __restrict__ h0, int T, int D, int nc,
                                                        long n_threads, const float* __restrict__ Plog,
                                                        const float* __restrict__ S, float* __restrict__ y,
                                                        float* __restrict__ h_final) {
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    if (g >= n_threads) return;
    const int DV = D / V;
    const int d = V * (int)(g % DV);
    const long rem = g / DV;
    const int ch = (int)(rem % nc);
    const long b = rem / nc;
    const int t0 = ch * kHawkChunk, t1 = min(T, t0 + kHawkChunk);
    float csp[V], h[V];
#pragma unroll
    for (int q = 0; q < V; ++q) {
        csp[q] = hawk_scale2(c, lam[d + q]);
        h[q] = h0 ? h0[b * D + d + q] : 0.f;
    }
    // the chunk's start state: fold the earlier chunks' (P, s) in order,
    // eight summaries requested at a time
    {
        const size_t j0 = (size_t)b * nc * D + d;
        int cc = 0;
        for (; cc + 8 <= ch; cc += 8) {
            HawkVec<float, V> pl[8], sv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                pl[u].load(Plog + j0 + (size_t)(cc + u) * D);
                sv[u].load(S + j0 + (size_t)(cc + u) * D);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u)
#pragma unroll
                for (int q = 0; q < V; ++q) h[q] = __builtin_amdgcn_exp2f(pl[u].get(q)) * h[q] + sv[u].get(q);
        }
        for (; cc < ch; ++cc) {
            HawkVec<float, V> pl, sv;
            pl.load(Plog + j0 + (size_t)cc * D);
            sv.load(S + j0 + (size_t)cc * D);
#pragma unroll
            for (int q = 0; q < V; ++q) h[q] = __builtin_amdgcn_exp2f(pl.get(q)) * h[q] + sv.get(q);
        }
    }
    size_t i = ((size_t)b * T + t0) * D + d;
    int t = t0;
    for (; t + kHawkUnroll <= t1; t += kHawkUnroll) {
        HawkVec<In, V> xr[kHawkUnroll], ar[kHawkUnroll], gr[kHawkUnroll];
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            xr[u].load(x + i + (size_t)u * D);
            ar[u].load(ga + i + (size_t)u * D);
            gr[u].load(gx + i + (size_t)u * D);
        }
#pragma unroll
        for (int u = 0; u < kHawkUnroll; ++u) {
            float out[V];
#pragma unroll
            for (int q = 0; q < V; ++q) {
                float la, av, vv;
                hawk_step_f(xr[u].get(q), ar[u].get(q), gr[u].get(q), csp[q], la, av, vv);
                h[q] = av * h[q] + vv;
                out[q] = h[q];
            }
            store_v<V>(y + i + (size_t)u * D, out);
        }
        i += (size_t)kHawkUnroll * D;
    }
    for (; t < t1; ++t, i += D) {
        HawkVec<In, V> xr, ar, gr;
        xr.load(x + i);
        ar.load(ga + i);
        gr.load(gx + i);
        float out[V];
#pragma unroll
        for (int q = 0; q < V; ++q) {
            float la, av, vv;
            hawk_step_f(xr.get(q), ar.get(q), gr.get(q), csp[q], la, av, vv);
            h[q] = av * h[q] + vv;
            out[q] = h[q];
        }
        store_v<V>(y + i, out);
    }
    if (h_final && ch == nc - 1) store_v<V>(h_final + b * D + d, h);
}

// One-pass schedule.  Lane l of every wave owns channel d = 64 blk + l of
// sequence b.  Inputs are read through buffer resources spanning the
// sequence, so the rows past its end (the next round's prefetch, a ragged
// last round, the lanes past D on the last row) read as zero without a
// fault; those steps are replaced by the identity (a = 1, u = 0).
template <typename In> struct HawkRaw;
template <> struct HawkRaw<float> {
    float v;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        v = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 2));
    }
    __device__ __forceinline__ float get() const { return v; }
};
template <> struct HawkRaw<bf16_t> {
    unsigned short v;
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
        v = __builtin_amdgcn_raw_buffer_load_b16(r, off, 0, 2);
    }
    __device__ __forceinline__ float get() const { return __uint_as_float((uint32_t)v << 16); }
};

#ifndef MESA_HAWK_WAVES
#define MESA_HAWK_WAVES 8
#endif
#ifndef MESA_HAWK_SEG
#define MESA_HAWK_SEG 8
#endif
constexpr int kHawkWaves = MESA_HAWK_WAVES;   // waves of a one-pass workgroup (segments per round)
constexpr int kHawkSeg = MESA_HAWK_SEG;       // tokens per wave per round

// A raw buffer resource of `bytes` bytes from base (capped at 2^32 - 1: the
// offsets used are far below that).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t hawk_rsrc(const void* base, size_t bytes) {
    const uint32_t n = bytes > 0xffffffffull ? 0xffffffffu : (uint32_t)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}

template <typename In, int R, int NW>
__global__ __launch_bounds__(64 * NW) void hawk_stream_kernel(const In* __restrict__ x, const In* __restrict__ ga,
                                                              const In* __restrict__ gx,
                                                              const float* __restrict__ lam, float c,
                                                              const float* __restrict__ h0, int T, int D,
                                                              int n_dblk, float* __restrict__ y,
                                                              float* __restrict__ h_final) {
    __shared__ float2 summ[2][NW][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int b = blockIdx.x / n_dblk;
    const int d = (blockIdx.x % n_dblk) * 64 + lane;
    const bool on = d < D;
    const float csp = on ? hawk_scale2(c, lam[d]) : 0.f;
    float carry = (on && h0) ? h0[(size_t)b * D + d] : 0.f;

    // Each round's rows are addressed through resources that start at the
    // round's first row and end at the sequence's end, so the per-lane byte
    // offsets stay the same from round to round.
    const size_t seq = (size_t)b * T * D, round_elems = (size_t)NW * R * D;
    const size_t in_bytes = (size_t)T * D * sizeof(In), y_bytes = (size_t)T * D * 4;
    const uint32_t row = (uint32_t)D * sizeof(In), yrow = (uint32_t)D * 4;
    const uint32_t off = (uint32_t)(w * R) * row + (uint32_t)d * sizeof(In);
    const uint32_t yoff = (uint32_t)(w * R) * yrow + (uint32_t)d * 4;
    auto rest = [](size_t total, size_t used) { return total > used ? total - used : 0; };

    // One round: prefetch the next round's rows into nxt, scan this wave's
    // segment from cur, exchange the segments' summaries, write the outputs.
    auto round = [&](HawkRaw<In>(&cur)[3][R], HawkRaw<In>(&nxt)[3][R], int rd) {
        {
            const size_t e = seq + (size_t)(rd + 1) * round_elems;
            const size_t nb = rest(in_bytes, (size_t)(rd + 1) * round_elems * sizeof(In));
            const __amdgpu_buffer_rsrc_t rx = hawk_rsrc(x + e, nb), ra = hawk_rsrc(ga + e, nb),
                                         rg = hawk_rsrc(gx + e, nb);
#pragma unroll
            for (int j = 0; j < R; ++j) {
                nxt[0][j].load(rx, off + j * row);
                nxt[1][j].load(ra, off + j * row);
                nxt[2][j].load(rg, off + j * row);
            }
        }
        const int t0 = rd * NW * R + w * R;
        // the segment's prefix decay products and states from zero; steps
        // past the sequence's end are the identity
        float pl[R], sl[R];
        float p = 1.f, s = 0.f;
        auto scan = [&](auto tail) {
#pragma unroll
            for (int j = 0; j < R; ++j) {
                float la, av, uv;
                hawk_step_f(cur[0][j].get(), cur[1][j].get(), cur[2][j].get(), csp, la, av, uv);
                if constexpr (decltype(tail)::value) {
                    if (t0 + j >= T) { av = 1.f; uv = 0.f; }
                }
                s = av * s + uv;
                p *= av;
                pl[j] = p;
                sl[j] = s;
            }
        };
        if (t0 + R <= T) scan(std::false_type{});
        else scan(std::true_type{});
        summ[rd & 1][w][lane] = float2{p, s};
        __syncthreads();
        // fold the earlier segments into this wave's start state, and all of
        // them into the next round's
        float cw = carry;
#pragma unroll
        for (int v = 0; v < NW; ++v) {
            const float2 e = summ[rd & 1][v][lane];
            if (v == w) cw = carry;
            carry = e.x * carry + e.y;
        }
        // rows past the sequence's end fall outside ry and are dropped
        const __amdgpu_buffer_rsrc_t ry =
            hawk_rsrc(y + seq + (size_t)rd * round_elems, rest(y_bytes, (size_t)rd * round_elems * 4));
        if (on) {
#pragma unroll
            for (int j = 0; j < R; ++j)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pl[j] * cw + sl[j]), ry,
                                                      yoff + j * yrow, 0, 2);
        }
    };

    HawkRaw<In> A[3][R], B[3][R];
    {
        const __amdgpu_buffer_rsrc_t rx = hawk_rsrc(x + seq, in_bytes), ra = hawk_rsrc(ga + seq, in_bytes),
                                     rg = hawk_rsrc(gx + seq, in_bytes);
#pragma unroll
        for (int j = 0; j < R; ++j) {
            A[0][j].load(rx, off + j * row);
            A[1][j].load(ra, off + j * row);
            A[2][j].load(rg, off + j * row);
        }
    }
    // an even number of rounds (a round past the end changes nothing), so
    // the two register sets alternate without copies
    const int n_rounds = 2 * ((T + 2 * NW * R - 1) / (2 * NW * R));
    for (int rd = 0; rd < n_rounds; rd += 2) {
        round(A, B, rd);
        round(B, A, rd + 1);
    }
    if (h_final && w == 0 && on) h_final[(size_t)b * D + d] = carry;
}

// The one-pass schedule needs enough 64-channel blocks to fill the GPU, and
// the byte offsets of a round's fp32 rows below 2^31.
static bool hawk_one_pass(const HawkArgs& a) {
    const long blocks = (long)a.B * ((a.D + 63) / 64);
    return blocks >= 128 && (size_t)kHawkWaves * kHawkSeg * a.D * 4 < (size_t(1) << 31);
}

template <typename In>
static hipError_t launch_stream_t(const HawkArgs& a, hipStream_t s) {
    const int n_dblk = (a.D + 63) / 64;
    hipLaunchKernelGGL((hawk_stream_kernel<In, kHawkSeg, kHawkWaves>), dim3((unsigned)(a.B * n_dblk)),
                       dim3(64 * kHawkWaves), 0, s, (const In*)a.x, (const In*)a.ga, (const In*)a.gx, a.lam, a.c,
                       a.h0, a.T, a.D, n_dblk, a.y, a.h_final);
    return hipGetLastError();
}

template <typename In, int V>
static hipError_t launch_t(const HawkArgs& a, hipStream_t s) {
    const long n = (long)a.B * a.nc * (a.D / V);
    const unsigned blocks = (unsigned)((n + 255) / 256);
    hipLaunchKernelGGL((hawk_summary_kernel<In, V>), dim3(blocks), dim3(256), 0, s, (const In*)a.x,
                       (const In*)a.ga, (const In*)a.gx, a.lam, a.c, a.T, a.D, a.nc, n, a.Plog, a.S);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((hawk_scan_kernel<In, V>), dim3(blocks), dim3(256), 0, s, (const In*)a.x, (const In*)a.ga,
                       (const In*)a.gx, a.lam, a.c, a.h0, a.T, a.D, a.nc, n, a.Plog, a.S, a.y, a.h_final);
    return hipGetLastError();
}

// One pass for wide shapes; else two passes with four channels per thread
// (one 8- or 16-byte piece per row) when the rows and pointers allow it, else
// one.
hipError_t launch_hawk(const HawkArgs& a, hipStream_t s) {
    if (hawk_one_pass(a)) return a.bf16 ? launch_stream_t<bf16_t>(a, s) : launch_stream_t<float>(a, s);
    const size_t esz = a.bf16 ? 2 : 4;
    auto al = [&](const void* p, size_t n) { return p == nullptr || reinterpret_cast<uintptr_t>(p) % n == 0; };
    const bool vec = a.D % 4 == 0 && al(a.x, 4 * esz) && al(a.ga, 4 * esz) && al(a.gx, 4 * esz) && al(a.y, 16) &&
                     al(a.h0, 16) && al(a.h_final, 16) && al(a.lam, 16) && al(a.Plog, 16) && al(a.S, 16);
    if (a.bf16) return vec ? launch_t<bf16_t, 4>(a, s) : launch_t<bf16_t, 1>(a, s);
    return vec ? launch_t<float, 4>(a, s) : launch_t<float, 1>(a, s);
}

}  // namespace mesa
