// bwd_states.hip -- the backward's reverse chunk states (gfx950).
//
// The backward of the Mesa layer (implicit differentiation of
// o_t = G_t (H_t + Lambda)^{-1} q_t; the page, section "A Camada Mesa",
// bullet "Paralelizacao", says the layer trains in parallel but gives no
// gradient) needs, for every key i, sums over the later tokens t >= i:
//   sum_t zeta_ti (x_t . k_i) g_t,   sum_t zeta_ti (g_t . v_i) x_t,
//   sum_t zeta_ti [(x_t . k_i) z_t + (z_t . k_i) x_t].
// Chunkwise, the tokens after chunk c enter through two d x d states
//   P^gx_c = sum_{t > e_c} e^{L_t - L_{e_c}} g_t x_t^T,   P^zx_c likewise with z_t,
// (e_c the chunk's last token, L the prefix sum of ln gamma), which obey,
// walking the chunks backwards with l the within-chunk prefix sums,
//   P_{c-1} = e^{l_end} P_c + sum_{t in c} e^{l_t} a_t x_t^T     (a = g or z).
// The key gradient needs P^zx only through its symmetric part, so this kernel
// produces P^gx_c and M_c = P^zx_c + (P^zx_c)^T for every chunk (both zero
// after the last chunk); M obeys the same recurrence with the rank-2C update
// sum_t e^{l_t} (z_t x_t^T + x_t z_t^T).  Work split as the forward's
// chunk-state kernel: one workgroup per (head, {gx, zx}, row block), each wave
// a 16 x D slab of the running state in MFMA accumulators, the update summed
// apart from it on MFMAs (two products per tile for M).  For d >= 32 the
// update runs on v_mfma_f32_16x16x32_f16 over two-part fp16 splits (cg_h2.h)
// of the chunk's token rows, a e^{l_t} and x each scaled by one power of two
// per chunk: three products per operand pair, so each product term carries
// about 22 significant bits; for d = 16 on v_mfma_f32_16x16x4_f32.
//
// States are stored as 16 x 16 blocks of 16 bytes per lane, each once per
// chunk in MFMA accumulator order (lane 16q + m holds rows 4q..4q+3 of
// column m).  Block (a, b) in that order is block (b, a) of the transpose in
// operand order (lane 16q + m holds columns 4q..4q+3 of row m): the key/value
// kernel reads P^gx's blocks so as rows of (P^gx)^T, and passes them through a
// per-wave LDS transpose for the rows of P^gx.  M, being symmetric, needs no
// transpose: its block (g, j) is its block (j, g) in operand order.  For
// d >= 32 a lane's 16 bytes are the two-part fp16 split (cg_h2.h) of its four
// values, hi then lo, scaled by 2^E with one exponent E per 16-row block
// (the wave's slab) and chunk, stored beside the states; for d = 16 the four
// floats themselves.
#include "cg_h2.h"
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

// The 16x16x32 fp16 MFMA operand of features c0 .. c0 + 15 (lane (m, kk):
// feature c0 + m) over tokens 32 s + 8 kk .. + 7, from an fp16 plane of token
// rows (pitch PW words), through two transposed 8-byte LDS reads (gfx950's
// ds_read_b64_tr_b16; lds_tr_f16x4 in cg_h2.h): lane m addresses token row
// r0 + m / 4 at the 4-feature piece c0 + 4 (m % 4) and receives feature
// c0 + m of rows r0 .. r0 + 3.  The A and B operands of an update read the
// same token order, so each k-slot is one token.
template <int PW>
__device__ __forceinline__ f16x8 token_plane_operand(const uint32_t* P, int c0, int s, int m, int kk) {
    const uint32_t* R = P + (c0 + 4 * (m & 3)) / 2;
    const f16x4 a = lds_tr_f16x4(R + (32 * s + 8 * kk + (m >> 2)) * PW);
    const f16x4 b = lds_tr_f16x4(R + (32 * s + 8 * kk + 4 + (m >> 2)) * PW);
    return f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

template <int D, int C, int NW>
__global__ __launch_bounds__(64 * NW) void bwd_states_kernel(
    const float* __restrict__ g, const float* __restrict__ z, const float* __restrict__ x,
    const float* __restrict__ gamma, int T, int n_chunks, float* __restrict__ Pgx, float* __restrict__ Pzx,
    int* __restrict__ Egx, int* __restrict__ Ezx, long BH) {
    constexpr int RB = D / (16 * NW);   // row blocks per state
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    constexpr int NTHR = 64 * NW;
    // d >= 32: the update on fp16 MFMAs over two-part splits, from token-row
    // planes of a_t e^{l_t} 2^Ea and x_t 2^Ex (one exponent per chunk and
    // tensor), padded to a whole 32-token step; d = 16: fp32 MFMAs from fp32
    // token rows
    constexpr bool H2 = D >= 32;
    constexpr int TR = C >= 32 ? C : 32;   // token rows of an fp16 plane
    constexpr int PW = D / 2 + 8;          // words per fp16 token row
    __shared__ float sA[H2 ? 4 : C * PD];   // g or z rows of the chunk (the state's rows)
    __shared__ float sX[H2 ? 4 : C * PD];   // x rows of the chunk (the state's columns)
    __shared__ alignas(16) uint32_t pA[2][H2 ? TR * PW : 4];   // (g or z) e^{l_t} 2^Ea: hi, lo
    __shared__ alignas(16) uint32_t pX[2][H2 ? TR * PW : 4];   // x 2^Ex: hi, lo
    __shared__ float sMax[2][NW];   // per-wave maxima of |a|, |x|
    __shared__ float sW[C];        // e^{l_t}
    __shared__ float sGam;         // e^{l_end}

    const int tid0 = threadIdx.x;
    const int lane = tid0 & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid0 >> 6);
    const int n = lane & 15;
    const int kk = lane >> 4;
    // XCD-aware id (as the forward's chunk-state kernel): consecutive ids go
    // round-robin over the 8 XCDs, so the 2*RB parts of head bh get ids
    // xcd + 8*(slot) with equal xcd and share that XCD's L2 for x (and the
    // g or z rows).
    constexpr int PARTS = 2 * RB;
    const long xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const long bh = (slot / PARTS) * 8 + xcd;
    const int part = (int)(slot % PARTS);
    if (bh >= BH) return;   // whole workgroup
    const int rb = part % RB;
    // 0: gx, 1: zx.  The kinds swap for every other group of eight heads on
    // an XCD, so that the two workgroups a CU takes in turn (ids 32 slots
    // apart on one XCD) are mostly one gx and one zx part: the zx parts do
    // twice the MFMA work.
    const int which = (part / RB) ^ (int)((slot / PARTS / 8) & 1);
    const int m0 = rb * 16 * NW + 16 * w;
    const float* ah = (which == 0 ? g : z) + (size_t)bh * T * D;
    const float* xh = x + (size_t)bh * T * D;
    const float* gh = gamma + (size_t)bh * T;
    const bool sym = which == 1;   // M = P^zx + (P^zx)^T
    const size_t pstride = (size_t)D * D;   // floats per chunk
    float* Pout = (which == 0 ? Pgx : Pzx) + (size_t)bh * n_chunks * pstride;
    int* Eout = (which == 0 ? Egx : Ezx) + (size_t)bh * n_chunks * NT;
    const int a0 = m0 / 16;        // the wave's row block

    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The next (earlier) chunk's rows and gates are held in registers while
    // this chunk's products run.  Lane-dependent addresses are rebuilt from an
    // opaque copy of the thread id in every step instead of being held across
    // the chunk loop (which would cost the second workgroup per CU).
    constexpr int EL4 = C * D / (4 * NTHR);   // 4-element groups per thread per tile
    static_assert(C * D % (4 * NTHR) == 0, "tile must split evenly over the workgroup");
    f32x4 areg[EL4], xreg[EL4];
    float greg = 1.0f;
    auto prefetch = [&](int c) {
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int t0 = c * C;
        const int valid = min(C, T - t0);
#pragma unroll
        for (int u = 0; u < EL4; ++u) {
            const int e = (tid + u * NTHR) * 4;
            const int i = e / D, f = e % D;
            areg[u] = xreg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < valid) {
                areg[u] = *reinterpret_cast<const f32x4*>(ah + (size_t)(t0 + i) * D + f);
                xreg[u] = *reinterpret_cast<const f32x4*>(xh + (size_t)(t0 + i) * D + f);
            }
        }
        if (w == 0) greg = lane < valid ? gh[t0 + lane] : 1.0f;
    };

    if constexpr (H2 && TR > C) {
        // the token rows past a 16-token chunk stay zero (covered by the
        // first chunk's barriers)
        for (int e = tid0; e < (TR - C) * PW; e += NTHR) {
            pA[0][C * PW + e] = pA[1][C * PW + e] = 0u;
            pX[0][C * PW + e] = pX[1][C * PW + e] = 0u;
        }
    }
    if (n_chunks > 0) prefetch(n_chunks - 1);
    for (int c = n_chunks - 1; c >= 0; --c) {
        int tid = tid0;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63, n = lane & 15, kk = lane >> 4;
        const int valid = min(C, T - c * C);
        f32x4 U[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) U[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        float su = 1.0f;   // undoes the planes' exponents
        if constexpr (H2) {
            // ---- (1) the chunk's maxima and log decays ----
            float am = 0.f, xm = 0.f;
#pragma unroll
            for (int u = 0; u < EL4; ++u)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    am = fmaxf(am, fabsf(areg[u][r]));
                    xm = fmaxf(xm, fabsf(xreg[u][r]));
                }
            am = wave_max(am);
            xm = wave_max(xm);
            if (lane == 0) {
                sMax[0][w] = am;
                sMax[1][w] = xm;
            }
            if (w == 0) {
                const float l = chunk_log_decay_of(greg, valid, lane);
                const float lend = __shfl(l, C - 1, 64);
                if (lane < C) sW[lane] = __expf(l);
                if (lane == 0) sGam = __expf(lend);
            }
            __syncthreads();
            float amax = 0.f, xmax = 0.f;
#pragma unroll
            for (int w2 = 0; w2 < NW; ++w2) {
                amax = fmaxf(amax, sMax[0][w2]);
                xmax = fmaxf(xmax, sMax[1][w2]);
            }
            const int Ea = h2_exp(amax), Ex = h2_exp(xmax);   // e^{l_t} <= 1 keeps |a e^{l_t}| <= max |a|
            const float sa = pow2(Ea), sx = pow2(Ex);
            su = pow2(-(Ea + Ex));
            // ---- (2) the planes: a thread's 4 features of token i, 8 bytes per plane ----
#pragma unroll
            for (int u = 0; u < EL4; ++u) {
                const int e = (tid + u * NTHR) * 4;
                const int i = e / D, f = e % D;
                const float wa = sW[i] * sa;
                f16x4 ah, al, xh, xl;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float ya = areg[u][r] * wa, yx = xreg[u][r] * sx;
                    ah[r] = (_Float16)ya;
                    al[r] = (_Float16)(ya - (float)ah[r]);
                    xh[r] = (_Float16)yx;
                    xl[r] = (_Float16)(yx - (float)xh[r]);
                }
                *reinterpret_cast<f16x4*>(&pA[0][i * PW + f / 2]) = ah;
                *reinterpret_cast<f16x4*>(&pA[1][i * PW + f / 2]) = al;
                *reinterpret_cast<f16x4*>(&pX[0][i * PW + f / 2]) = xh;
                *reinterpret_cast<f16x4*>(&pX[1][i * PW + f / 2]) = xl;
            }
            __syncthreads();
            if (c > 0) prefetch(c - 1);

            // ---- (3) U = sum_t (a_t e^{l_t}) x_t^T over the wave's 16 rows; M also
            //      gains sum_t x_t (a_t e^{l_t})^T: three fp16 products per operand pair ----
            // each 32-token step and column block a fresh three-product chain
            // (from zero, read only after it), added into U on the VALU: longer
            // chains got accumulator inputs rewritten a few wait states after issue
            const f32x4 zero = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int st = 0; st < TR / 32; ++st) {
                const f16x8 Ah = token_plane_operand<PW>(pA[0], m0, st, n, kk);
                const f16x8 Al = token_plane_operand<PW>(pA[1], m0, st, n, kk);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    const f16x8 Bh = token_plane_operand<PW>(pX[0], 16 * j, st, n, kk);
                    const f16x8 Bl = token_plane_operand<PW>(pX[1], 16 * j, st, n, kk);
                    f32x4 t = mfma_f16x32(Al, Bh, zero);
                    t = mfma_f16x32(Ah, Bl, t);
                    t = mfma_f16x32(Ah, Bh, t);
                    U[j] += t;
                }
                if (sym) {
                    // M's transposed products
                    const f16x8 Xh = token_plane_operand<PW>(pX[0], m0, st, n, kk);
                    const f16x8 Xl = token_plane_operand<PW>(pX[1], m0, st, n, kk);
#pragma unroll
                    for (int j = 0; j < NT; ++j) {
                        const f16x8 Ch = token_plane_operand<PW>(pA[0], 16 * j, st, n, kk);
                        const f16x8 Cl = token_plane_operand<PW>(pA[1], 16 * j, st, n, kk);
                        f32x4 t = mfma_f16x32(Xl, Ch, zero);
                        t = mfma_f16x32(Xh, Cl, t);
                        t = mfma_f16x32(Xh, Ch, t);
                        U[j] += t;
                    }
                }
            }
        } else {
#pragma unroll
            for (int u = 0; u < EL4; ++u) {
                const int e = (tid + u * NTHR) * 4;
                const int i = e / D, f = e % D;
                *reinterpret_cast<f32x4*>(&sA[i * PD + f]) = areg[u];
                *reinterpret_cast<f32x4*>(&sX[i * PD + f]) = xreg[u];
            }
            if (w == 0) {
                const float l = chunk_log_decay_of(greg, valid, lane);
                const float lend = __shfl(l, C - 1, 64);
                if (lane < C) sW[lane] = __expf(l);
                if (lane == 0) sGam = __expf(lend);
            }
            __syncthreads();
            if (c > 0) prefetch(c - 1);

            // ---- P <- e^{l_end} P + sum_t e^{l_t} a_t x_t^T  (U a fresh MFMA chain);
            //      M also gains sum_t e^{l_t} x_t z_t^T ----
#pragma unroll
            for (int gg = 0; gg < C / 16; ++gg) {
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int i = 16 * gg + 4 * kk + s;
                    const float a = sA[i * PD + m0 + n] * sW[i];
#pragma unroll
                    for (int j = 0; j < NT; ++j) U[j] = mfma4(a, sX[i * PD + 16 * j + n], U[j]);
                }
            }
            if (sym) {
#pragma unroll
                for (int gg = 0; gg < C / 16; ++gg) {
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        const int i = 16 * gg + 4 * kk + s;
                        const float a = sX[i * PD + m0 + n] * sW[i];
#pragma unroll
                        for (int j = 0; j < NT; ++j) U[j] = mfma4(a, sA[i * PD + 16 * j + n], U[j]);
                    }
                }
            }
        }
        // ---- the state of the tokens after this chunk, blocks (a0, j): stored
        //      while the update's MFMAs run ----
        {
            float* dst = Pout + (size_t)c * pstride + 4 * lane;
            if constexpr (D >= 32) {
                const int E = h2_exp(wave_max(absmax<NT>(acc)));
                const float sc = pow2(E);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
                    f16x4 h, l;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const float y = acc[j][r] * sc;
                        h[r] = (_Float16)y;
                        l[r] = (_Float16)(y - (float)h[r]);
                    }
                    typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));
                    const u32x2v hw = __builtin_bit_cast(u32x2v, h), lw = __builtin_bit_cast(u32x2v, l);
                    store_nt(dst + (a0 * NT + j) * 256,
                             f32x4{__uint_as_float(hw[0]), __uint_as_float(hw[1]), __uint_as_float(lw[0]),
                                   __uint_as_float(lw[1])});
                }
                if (lane == 0) Eout[(size_t)c * NT + a0] = E;
            } else {
#pragma unroll
                for (int j = 0; j < NT; ++j) store_nt(dst + (a0 * NT + j) * 256, acc[j]);
            }
        }

        const float G = sGam;
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] = G * acc[j] + su * U[j];
        __syncthreads();
    }
}

template <int D, int C>
static hipError_t launch_t(const BwdStatesArgs& a, hipStream_t s) {
    constexpr int NW = D >= 64 ? 4 : D / 16;
    constexpr int RB = D / (16 * NW);
    const long grid = ((a.BH + 7) / 8) * 8 * 2 * RB;   // heads rounded up to a multiple of 8
    hipLaunchKernelGGL((bwd_states_kernel<D, C, NW>), dim3((unsigned)grid), dim3(64 * NW), 0, s, a.g, a.z, a.x,
                       a.gamma, a.T, a.n_chunks, a.Pgx, a.Pzx, a.Egx, a.Ezx, a.BH);
    return hipGetLastError();
}

template <int D>
static hipError_t dispatch_c(const BwdStatesArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_t<D, 16>(a, s);
        case 32: return launch_t<D, 32>(a, s);
        case 64: return launch_t<D, 64>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_states(const BwdStatesArgs& a, hipStream_t s) {
    switch (a.d) {
        case 16: return dispatch_c<16>(a, s);
        case 32: return dispatch_c<32>(a, s);
        case 64: return dispatch_c<64>(a, s);
        case 128: return dispatch_c<128>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace mesa
