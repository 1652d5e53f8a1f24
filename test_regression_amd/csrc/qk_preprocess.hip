// qk_preprocess.hip -- query/key pre-processing before the Mesa layer (gfx950).
//
// MesaNet summary page (gist.science, paper 2506.05233), section
// "Arquitetura (MesaNet)", bullet "Pre-processamento": keys and queries are
// normalised and convolved with a small window before the Mesa layer.
// Per head h, token t and feature f (W the window, at most 4 here):
//   c_t[f] = sum_{j<W} w[h][j][f] x_{t-j}[f]     (rows before t = 0 from hist)
//   y_t    = c_t / |c_t|_2                       (0 when c_t = 0)
// The convolution, the normalisation and the output cast happen in one pass:
// HBM traffic is one read of x and one write of y.
//
// Work split: a thread owns F consecutive features (16 bytes of input) of
// one head over a segment of L consecutive tokens; the G = d/F threads of a
// segment are adjacent lanes, so each token row is read as one contiguous
// piece and its norm is a reduction over those lanes (every lane adds the
// same two operands, so all of them scale by the same value).  The thread
// keeps the window's earlier rows and its weights in registers and walks its
// segment U tokens at a time, loading the U rows before using them; only the
// W-1 rows before a segment are read twice.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

constexpr int kPreMaxWidth = kQkPreMaxWidth;
constexpr int kPreSegment = kQkPreSegment;   // tokens per thread
#ifndef MESA_QK_PRE_UNROLL
#define MESA_QK_PRE_UNROLL 4
#endif
constexpr int kPreUnroll = MESA_QK_PRE_UNROLL;   // tokens loaded together

// Two float32 -> packed bfloat16 pair, round to nearest even (v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pack_rne(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2_t));
}

// F consecutive values of one row, as float.
template <int F>
struct Vec { float v[F]; };

__device__ __forceinline__ Vec<4> loadv(const float* p) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(p);
    return Vec<4>{{a[0], a[1], a[2], a[3]}};
}
__device__ __forceinline__ Vec<8> loadv(const bf16_t* p) {
    const uint4 u = *reinterpret_cast<const uint4*>(p);
    Vec<8> r;
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        r.v[2 * i] = __uint_as_float(w[i] << 16);
        r.v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
    return r;
}
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
template <int F>
__device__ __forceinline__ void storev(float* p, const Vec<F>& a) {
#pragma unroll
    for (int i = 0; i < F; i += 4)
        __builtin_nontemporal_store(f32x4{a.v[i], a.v[i + 1], a.v[i + 2], a.v[i + 3]}, reinterpret_cast<f32x4*>(p + i));
}
template <int F>
__device__ __forceinline__ void storev(bf16_t* p, const Vec<F>& a) {
    uint32_t w[F / 2];
#pragma unroll
    for (int i = 0; i < F / 2; ++i) w[i] = bf16_pack_rne(a.v[2 * i], a.v[2 * i + 1]);
    if constexpr (F == 8) __builtin_nontemporal_store(u32x4_t{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4_t*>(p));
    else __builtin_nontemporal_store(u32x2_t{w[0], w[1]}, reinterpret_cast<u32x2_t*>(p));
}

// Sum over the G adjacent lanes of a token row (G a power of two <= 32).
template <int G>
__device__ __forceinline__ float row_group_sum(float v) {
    if constexpr (G >= 2) v += dpp<0xB1>(v);    // quad_perm [1,0,3,2]
    if constexpr (G >= 4) v += dpp<0x4E>(v);    // quad_perm [2,3,0,1]
    if constexpr (G >= 8) v += dpp<0x141>(v);   // row_half_mirror
    if constexpr (G >= 16) v += dpp<0x140>(v);  // row_mirror
    if constexpr (G >= 32) {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    }
    return v;
}

template <int D, typename In, typename Out>
__global__ __launch_bounds__(256) void qk_preprocess_kernel(const In* __restrict__ x, const float* __restrict__ w,
                                                            int W, const In* __restrict__ hist, int H, int T,
                                                            int segs_per_bh, long n_segs, Out* __restrict__ y) {
    constexpr int F = 16 / (int)sizeof(In);   // features per thread
    constexpr int G = D / F;                  // threads per token row
    constexpr int WM = kPreMaxWidth;
    constexpr int U = kPreUnroll;
    const long g = (long)blockIdx.x * 256 + threadIdx.x;
    const long seg = g / G;                   // uniform over a row's G lanes
    const bool live = seg < n_segs;
    const int f0 = F * (int)(g % G);
    const long bh = live ? seg / segs_per_bh : 0;
    const int t0 = live ? (int)(seg % segs_per_bh) * kPreSegment : 0;
    const int t1 = live ? min(T, t0 + kPreSegment) : 0;
    const int h = (int)(bh % H);
    const int HW = W - 1;
    const In* xb = x + (size_t)bh * T * D + f0;

    Vec<F> wr[WM];   // taps at or beyond W are zero
#pragma unroll
    for (int j = 0; j < WM; ++j)
#pragma unroll
        for (int i = 0; i < F; i += 4) {
            const f32x4 a = (live && j < W) ? *reinterpret_cast<const f32x4*>(w + ((size_t)h * W + j) * D + f0 + i)
                                            : f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int u = 0; u < 4; ++u) wr[j].v[i + u] = a[u];
        }
    Vec<F> prev[WM - 1];   // prev[j] = row t - 1 - j
#pragma unroll
    for (int j = 0; j < WM - 1; ++j) {
        const int src = t0 - 1 - j;
        Vec<F> z;
#pragma unroll
        for (int i = 0; i < F; ++i) z.v[i] = 0.f;
        if (live && j < HW) {
            if (src >= 0) z = loadv(xb + (size_t)src * D);
            else if (hist) z = loadv(hist + ((size_t)bh * HW + HW + src) * D + f0);
        }
        prev[j] = z;
    }

    for (int t = t0; t < t1; t += U) {   // t1 is uniform over a row's lanes; rows past t1 are masked
        Vec<F> cur[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (t + u < t1) {
                cur[u] = loadv(xb + (size_t)(t + u) * D);
            } else {
#pragma unroll
                for (int i = 0; i < F; ++i) cur[u].v[i] = 0.f;
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            Vec<F> c;
            float ss = 0.f;
#pragma unroll
            for (int i = 0; i < F; ++i) {
                float a = wr[0].v[i] * cur[u].v[i];
#pragma unroll
                for (int j = 1; j < WM; ++j) a += wr[j].v[i] * (j <= u ? cur[u - j].v[i] : prev[j - u - 1].v[i]);
                c.v[i] = a;
                ss += a * a;
            }
            ss = row_group_sum<G>(ss);
            const float nrm = sqrtf(ss);
            const float inv = nrm > 0.f ? 1.0f / nrm : 0.f;
#pragma unroll
            for (int i = 0; i < F; ++i) c.v[i] *= inv;
            if (t + u < t1) storev(y + ((size_t)bh * T + t + u) * D + f0, c);
        }
#pragma unroll
        for (int j = WM - 2; j >= 0; --j) prev[j] = j < U ? cur[U - 1 - j] : prev[j - U];
    }
}

// hist_out[r] = row T + r of [hist (W-1 rows); x (T rows)], for r < W - 1.
template <typename In>
__global__ __launch_bounds__(256) void qk_history_kernel(const In* __restrict__ x, const In* __restrict__ hist,
                                                         In* __restrict__ hist_out, int W, int T, int D,
                                                         long n_elems) {
    const long e = (long)blockIdx.x * 256 + threadIdx.x;
    if (e >= n_elems) return;
    const int HW = W - 1;
    const int f = (int)(e % D);
    const long rowi = e / D;
    const int r = (int)(rowi % HW);
    const long bh = rowi / HW;
    const int src = T - HW + r;   // position in x; < 0 reaches into hist
    In v{};
    if (src >= 0) v = x[((size_t)bh * T + src) * D + f];
    else if (hist) v = hist[((size_t)bh * HW + HW + src) * D + f];
    hist_out[e] = v;
}

template <int D, typename In, typename Out>
static hipError_t launch_t(const QkPreArgs& a, hipStream_t s) {
    if (a.n_segs > 0) {
        const long threads = a.n_segs * (D / (16 / (int)sizeof(In)));
        hipLaunchKernelGGL((qk_preprocess_kernel<D, In, Out>), dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, s, (const In*)a.x, a.w, a.W, (const In*)a.hist, a.H, a.T, a.segs_per_bh,
                           a.n_segs, (Out*)a.y);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (a.hist_out) {
        hipLaunchKernelGGL((qk_history_kernel<In>), dim3((unsigned)((a.n_hist + 255) / 256)), dim3(256), 0, s,
                           (const In*)a.x, (const In*)a.hist, (In*)a.hist_out, a.W, a.T, D, a.n_hist);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <typename In, typename Out>
static hipError_t dispatch_d(const QkPreArgs& a, hipStream_t s) {
    switch (a.d) {
        case 16: return launch_t<16, In, Out>(a, s);
        case 32: return launch_t<32, In, Out>(a, s);
        case 64: return launch_t<64, In, Out>(a, s);
        case 128: return launch_t<128, In, Out>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_qk_preprocess(const QkPreArgs& a, hipStream_t s) {
    if (a.in_bf16) return a.out_bf16 ? dispatch_d<bf16_t, bf16_t>(a, s) : dispatch_d<bf16_t, float>(a, s);
    return a.out_bf16 ? dispatch_d<float, bf16_t>(a, s) : dispatch_d<float, float>(a, s);
}

}  // namespace mesa
