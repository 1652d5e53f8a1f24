// bwd_kv.hip -- the backward's key and value gradients (gfx950).
//
// Implicit differentiation of o_t = G_t (H_t + Lambda)^{-1} q_t (the page,
// section "A Camada Mesa", bullet "Paralelizacao", says the layer trains in
// parallel but gives no gradient), at the forward's solutions x_t and the
// adjoint solutions z_t, for a loss with dL/do_t = g_t:
//   dL/dv_i = sum_{t>=i} zeta_ti (x_t . k_i) g_t
//   dL/dk_i = sum_{t>=i} zeta_ti [(g_t . v_i) x_t - (x_t . k_i) z_t - (z_t . k_i) x_t]
//   a_i     = (v_i . dL/dv_i + k_i . dL/dk_i) / 2      (the key-side gate total)
// Chunkwise, for key i of chunk c (l the within-chunk prefix sums, e_c the
// chunk's last token), the later chunks enter through the reverse states:
//   dv_i = sum_{t in c, t>=i} e^{l_t - l_i} (x_t . k_i) g_t + e^{l_e - l_i} P^gx_c k_i
//   dk_i = sum_{t in c, t>=i} e^{l_t - l_i} [(g_t . v_i - z_t . k_i) x_t - (x_t . k_i) z_t]
//          + e^{l_e - l_i} [(P^gx_c)^T v_i - (P^zx_c + (P^zx_c)^T) k_i]
// Work split: one workgroup per (head, chunk); wave w owns keys 16w..16w+15
// and holds their k_i, v_i in registers as the MFMA B operand (lane (n, kk):
// features 16j + 4kk + r of key n).  Scores come out of the MFMA in exactly
// the layout the next contraction (over tokens) takes as its B operand, so
// the token tiles are the A operand both ways: read along rows for the
// scores and down columns for the sums over tokens.  Then the two states
// replace the token tiles in LDS.  Every MFMA chain starts from zero and is
// only read afterwards.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

template <int D, int C>
struct alignas(16) KvLds {
    static constexpr int PD = lds_pitch(D);
    static constexpr int PS = lds_pitch_rows(D);
    static constexpr int TILES = 3 * C * PD;    // x, z, g rows of the chunk
    static constexpr int STATES = 2 * D * PS;   // P^gx, P^zx rows
    float R[TILES > STATES ? TILES : STATES];
    float L[C];
};

__device__ __forceinline__ f32x4 ld4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }

// Sc[tb] = A[16tb + m][:] . Z^T[:][n]: scores of the chunk's token rows
// (tile rows, pitch lds_pitch(D)) against the wave's keys or values in registers.
template <int D>
__device__ __forceinline__ f32x4 token_scores(const float* rows, const f32x4 (&Z)[D / 16], int m, int kk) {
    constexpr int NT = D / 16;
    constexpr int PD = lds_pitch(D);
    const float* a = rows + m * PD + 4 * kk;
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 buf[2];
    buf[0] = ld4(a);
#pragma unroll
    for (int gg = 0; gg < NT; ++gg) {
        if (gg + 1 < NT) buf[(gg + 1) & 1] = ld4(a + 16 * (gg + 1));
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = mfma4(buf[gg & 1][s], Z[gg][s], acc);
    }
    return acc;
}

// Y[j] += S[16j + m][:] . Z^T[:][n] for j in [J0, J0 + NJ) (ROWS), or
// S[:][16j + m] . Z^T[:][n] (columns), or (S + S^T)[16j + m][:] . Z^T[:][n]
// (SYM); S a full d x d state in LDS (pitch lds_pitch_rows(D)).  The output
// blocks go in groups so that their A operands and accumulators fit in
// registers.
template <int D, int MODE, int J0, int NJ>   // MODE 0: rows, 1: columns, 2: rows + columns
__device__ __forceinline__ void state_apply_part(const float* S, const f32x4 (&Z)[D / 16], int m, int kk,
                                                 f32x4 (&Y)[D / 16]) {
    constexpr int NT = D / 16;
    constexpr int PS = lds_pitch_rows(D);
#pragma unroll
    for (int gg = 0; gg < NT; ++gg) {
        f32x4 a[NJ];
#pragma unroll
        for (int jj = 0; jj < NJ; ++jj) {
            const int j = J0 + jj;
            if constexpr (MODE != 1) a[jj] = ld4(S + (16 * j + m) * PS + 16 * gg + 4 * kk);
            else a[jj] = f32x4{0.f, 0.f, 0.f, 0.f};
            if constexpr (MODE != 0) {
#pragma unroll
                for (int s = 0; s < 4; ++s) a[jj][s] += S[(16 * gg + 4 * kk + s) * PS + 16 * j + m];
            }
        }
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int jj = 0; jj < NJ; ++jj) Y[J0 + jj] = mfma4(a[jj][s], Z[gg][s], Y[J0 + jj]);
    }
}

template <int D, int MODE>
__device__ __forceinline__ void state_apply(const float* S, const f32x4 (&Z)[D / 16], int m, int kk,
                                            f32x4 (&Y)[D / 16]) {
    constexpr int NT = D / 16;
    constexpr int NJ = NT >= 4 ? NT / 2 : NT;
    state_apply_part<D, MODE, 0, NJ>(S, Z, m, kk, Y);
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (NJ < NT) state_apply_part<D, MODE, NJ, NT - NJ>(S, Z, m, kk, Y);
}

template <int D, int C, int W, typename In>
__device__ __forceinline__ void kv_wave(KvLds<D, C>& L, int lane, const In* __restrict__ k,
                                        const In* __restrict__ v, size_t tok0, int valid,
                                        const float* __restrict__ Pgx, const float* __restrict__ Pzx, int tid,
                                        float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ akey) {
    constexpr int NT = D / 16;
    constexpr int NW = C / 16;
    constexpr int PD = lds_pitch(D);
    constexpr int PS = lds_pitch_rows(D);
    constexpr int NTHR = 64 * NW;
    const int n = lane & 15, kk = lane >> 4;
    const int il = 16 * W + n;          // chunk-local key index of the lane
    const bool key_ok = il < valid;
    const float* X = L.R;
    const float* Zt = L.R + C * PD;
    const float* Gt = L.R + 2 * C * PD;

    f32x4 Kb[NT], Vb[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const size_t off = (tok0 + il) * D + 16 * j + 4 * kk;
        Kb[j] = key_ok ? load4(k + off) : f32x4{0.f, 0.f, 0.f, 0.f};
        Vb[j] = key_ok ? load4(v + off) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    const float li = L.L[il];

    // ---- within the chunk: tokens t >= i, one 16-token block at a time ----
    // Each block's sums are fresh MFMA chains, added into DK, DV on the VALU;
    // dk's pass and dv's pass run one after the other (register pressure).
    f32x4 DV[NT], DK[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) DV[j] = DK[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int tb = W; tb < NW; ++tb) {
        const f32x4 s1 = token_scores<D>(X + 16 * tb * PD, Kb, n, kk);    // x_t . k_i
        const f32x4 s2 = token_scores<D>(Gt + 16 * tb * PD, Vb, n, kk);   // g_t . v_i
        const f32x4 s3 = token_scores<D>(Zt + 16 * tb * PD, Kb, n, kk);   // z_t . k_i
        f32x4 w23, wn1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tb + 4 * kk + r;
            const float zeta = (t >= il) ? __expf(L.L[t] - li) : 0.f;
            w23[r] = zeta * (s2[r] - s3[r]);
            wn1[r] = -zeta * s1[r];
        }
        f32x4 BK[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) BK[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = 16 * tb + 4 * kk + s;
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                BK[j] = mfma4(X[t * PD + 16 * j + n], w23[s], BK[j]);
                BK[j] = mfma4(Zt[t * PD + 16 * j + n], wn1[s], BK[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) DK[j] += BK[j];
    }
#pragma unroll 1
    for (int tb = W; tb < NW; ++tb) {
        const f32x4 s1 = token_scores<D>(X + 16 * tb * PD, Kb, n, kk);    // x_t . k_i
        f32x4 w1;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int t = 16 * tb + 4 * kk + r;
            w1[r] = (t >= il) ? __expf(L.L[t] - li) * s1[r] : 0.f;
        }
        f32x4 BV[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) BV[j] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int t = 16 * tb + 4 * kk + s;
#pragma unroll
            for (int j = 0; j < NT; ++j) BV[j] = mfma4(Gt[t * PD + 16 * j + n], w1[s], BV[j]);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) DV[j] += BV[j];
    }

    // ---- the later chunks, through the reverse states ----
    __syncthreads();   // every wave is done with the token tiles
    {
        const float* src[2] = {Pgx, Pzx};
        for (int e = tid * 4; e < 2 * D * D; e += NTHR * 4) {
            const int which = e / (D * D), r = (e % (D * D)) / D, f = e % D;
            *reinterpret_cast<f32x4*>(&L.R[which * D * PS + r * PS + f]) =
                *reinterpret_cast<const f32x4*>(src[which] + (size_t)r * D + f);
        }
    }
    __syncthreads();
    const float* SGX = L.R;
    const float* SZX = L.R + D * PS;
    const float es = __expf(L.L[C - 1] - li);   // e^{l_end - l_i}
    float vd = 0.f, kd = 0.f;
    {
        f32x4 A1[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) A1[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        state_apply<D, 0>(SGX, Kb, n, kk, A1);   // P^gx k_i
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                o[r] = DV[j][r] + es * A1[j][r];
                vd += Vb[j][r] * o[r];
            }
            if (key_ok) *reinterpret_cast<f32x4*>(dv + (tok0 + il) * D + 16 * j + 4 * kk) = o;
        }
    }
    {
        f32x4 A2[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) A2[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        state_apply<D, 1>(SGX, Vb, n, kk, A2);   // (P^gx)^T v_i
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) DK[j][r] += es * A2[j][r];
    }
    {
        f32x4 A3[NT];
#pragma unroll
        for (int j = 0; j < NT; ++j) A3[j] = f32x4{0.f, 0.f, 0.f, 0.f};
        state_apply<D, 2>(SZX, Kb, n, kk, A3);   // (P^zx + P^zx^T) k_i
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            f32x4 o;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                o[r] = DK[j][r] - es * A3[j][r];
                kd += Kb[j][r] * o[r];
            }
            if (key_ok) *reinterpret_cast<f32x4*>(dk + (tok0 + il) * D + 16 * j + 4 * kk) = o;
        }
    }
    const float a = 0.5f * (kslot_sum(vd) + kslot_sum(kd));
    if (key_ok && kk == 0) akey[tok0 + il] = a;
}

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (C / 16)) void bwd_kv_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma,
    const float* __restrict__ x, const float* __restrict__ z, const float* __restrict__ gout,
    const float* __restrict__ Pgx, const float* __restrict__ Pzx, int T, int n_chunks,
    float* __restrict__ dk, float* __restrict__ dv, float* __restrict__ akey) {
    constexpr int NW = C / 16;
    constexpr int PD = lds_pitch(D);
    constexpr int NTHR = 64 * NW;
    __shared__ KvLds<D, C> L;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x % n_chunks;
    const long bh = blockIdx.x / n_chunks;
    const int t0 = c * C;
    const int valid = min(C, T - t0);
    const size_t tok0 = (size_t)bh * T + t0;
    const size_t soff = ((size_t)bh * n_chunks + c) * D * D;

    // ---- x, z, g rows of the chunk; l ----
    const float* srcs[3] = {x, z, gout};
    for (int e = tid * 4; e < 3 * C * D; e += NTHR * 4) {
        const int which = e / (C * D), i = (e % (C * D)) / D, f = e % D;
        f32x4 val = f32x4{0.f, 0.f, 0.f, 0.f};
        if (i < valid) val = *reinterpret_cast<const f32x4*>(srcs[which] + (tok0 + i) * D + f);
        *reinterpret_cast<f32x4*>(&L.R[which * C * PD + i * PD + f]) = val;
    }
    if (w == 0) {
        const float l = chunk_log_decay(gamma + tok0, valid, lane);
        if (lane < C) L.L[lane] = l;
    }
    __syncthreads();

    const float* pg = Pgx + soff;
    const float* pz = Pzx + soff;
    if (w == 0) {
        kv_wave<D, C, 0, In>(L, lane, k, v, tok0, valid, pg, pz, tid, dk, dv, akey);
    } else if constexpr (NW > 1) {
        if (w == 1) {
            kv_wave<D, C, 1, In>(L, lane, k, v, tok0, valid, pg, pz, tid, dk, dv, akey);
        } else if constexpr (NW > 2) {
            if (w == 2) kv_wave<D, C, 2, In>(L, lane, k, v, tok0, valid, pg, pz, tid, dk, dv, akey);
            else kv_wave<D, C, 3, In>(L, lane, k, v, tok0, valid, pg, pz, tid, dk, dv, akey);
        }
    }
}

template <int D, int C, typename In>
static hipError_t launch_t(const BwdKvArgs& a, hipStream_t s) {
    const long grid = a.BH * a.n_chunks;
    hipLaunchKernelGGL((bwd_kv_kernel<D, C, In>), dim3((unsigned)grid), dim3(64 * (C / 16)), 0, s, (const In*)a.k,
                       (const In*)a.v, a.gamma, a.x, a.z, a.gout, a.Pgx, a.Pzx, a.T, a.n_chunks, a.dk, a.dv, a.akey);
    return hipGetLastError();
}

template <int D, typename In>
static hipError_t dispatch_c(const BwdKvArgs& a, hipStream_t s) {
    switch (a.chunk) {
        case 16: return launch_t<D, 16, In>(a, s);
        case 32: return launch_t<D, 32, In>(a, s);
        case 64: return launch_t<D, 64, In>(a, s);
    }
    return hipErrorInvalidValue;
}

template <typename In>
static hipError_t dispatch_d(const BwdKvArgs& a, hipStream_t s) {
    switch (a.d) {
        case 16: return dispatch_c<16, In>(a, s);
        case 32: return dispatch_c<32, In>(a, s);
        case 64: return dispatch_c<64, In>(a, s);
        case 128: return dispatch_c<128, In>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_bwd_kv(const BwdKvArgs& a, hipStream_t s) {
    return a.bf16 ? dispatch_d<bf16_t>(a, s) : dispatch_d<float>(a, s);
}

}  // namespace mesa
