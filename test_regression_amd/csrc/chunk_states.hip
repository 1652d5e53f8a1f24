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
// Both states are stored row-major ([d][d_k], rows are key features for H
// and value features for G), the layout of the exported final states.
//
// Work split: one workgroup per (head, {H, G}, 16*NW-row block of the
// state); each wave holds a 16 x D slab of the running state in MFMA
// accumulator layout and walks the chunks in order.  Per chunk the update is
// one (16 x C) x (C x D) product on v_mfma_f32_16x16x4_f32 with the weighted
// rows (keys for H, values for G) as the A operand and the keys as the B
// operand; the contraction runs over the chunk's tokens.  Workgroup ids are
// mapped so that the 2*RB workgroups of one head land on the same XCD (ids
// congruent mod 8) and share its L2 for the key and value tiles.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

template <int D, int C, typename In>
__global__ __launch_bounds__(64 * (D >= 64 ? 4 : D / 16)) void chunk_states_kernel(
    const In* __restrict__ k, const In* __restrict__ v, const float* __restrict__ gamma,
    int T, int n_chunks, float* __restrict__ SH, float* __restrict__ SG,
    float* __restrict__ final_H, float* __restrict__ final_G, int write_chunks, long BH) {
    constexpr int NW = D >= 64 ? 4 : D / 16;   // waves per workgroup
    constexpr int RB = D / (16 * NW);          // row blocks per state
    constexpr int NT = D / 16;                 // 16-column tiles of the state
    constexpr int PD = lds_pitch(D);
    constexpr int NTHR = 64 * NW;

    __shared__ float sK[C * PD];   // keys of the chunk (B operand; A rows for H)
    __shared__ float sB[C * PD];   // values of the chunk (A rows for G)
    __shared__ float sW[C];        // e^{l_end - l_i}
    __shared__ float sGam;         // e^{l_end}

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int n = lane & 15;
    const int kk = lane >> 4;

    // XCD-aware id: consecutive ids go round-robin over the 8 XCDs, so the
    // 2*RB parts of head bh get ids xcd + 8*(slot) with equal xcd.
    constexpr int PARTS = 2 * RB;
    const long xcd = blockIdx.x % 8, slot = blockIdx.x / 8;
    const long bh = (slot / PARTS) * 8 + xcd;
    const int part = (int)(slot % PARTS);
    if (bh >= BH) return;                      // whole workgroup: no barrier is skipped
    const int rb = part % RB;
    const int which = part / RB;               // 0: H, 1: G
    const int m0 = rb * 16 * NW + 16 * w;      // first state row of this wave

    const In* kh = k + (size_t)bh * T * D;
    const In* vh = v + (size_t)bh * T * D;
    const float* gh = gamma + (size_t)bh * T;
    float* Sout = (which == 0 ? SH : SG) + (size_t)bh * n_chunks * D * D;
    const float* sArows = which == 0 ? sK : sB;

    f32x4 acc[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The next chunk's keys, values and gates are loaded into registers while
    // the current chunk's MFMAs run (global latency hidden behind compute).
    constexpr int EL4 = C * D / (4 * NTHR);   // 4-element groups per thread per tile
    static_assert(C * D % (4 * NTHR) == 0, "tile must split evenly over the workgroup");
    f32x4 kreg[EL4], vreg[EL4];
    float greg = 1.0f;
    auto prefetch = [&](int c) {
        const int t0 = c * C;
        const int valid = min(C, T - t0);
#pragma unroll
        for (int u = 0; u < EL4; ++u) {
            const int e = (tid + u * NTHR) * 4;
            const int i = e / D, f = e % D;
            kreg[u] = vreg[u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (i < valid) {
                kreg[u] = load4(kh + (size_t)(t0 + i) * D + f);
                if (which) vreg[u] = load4(vh + (size_t)(t0 + i) * D + f);
            }
        }
        if (w == 0) greg = lane < valid ? gh[t0 + lane] : 1.0f;
    };
    if (n_chunks > 0) prefetch(0);

    for (int c = 0; c < n_chunks; ++c) {
        // ---- stage the chunk's keys (and values) in LDS as fp32 ----
#pragma unroll
        for (int u = 0; u < EL4; ++u) {
            const int e = (tid + u * NTHR) * 4;
            const int i = e / D, f = e % D;
            *reinterpret_cast<f32x4*>(&sK[i * PD + f]) = kreg[u];
            if (which) *reinterpret_cast<f32x4*>(&sB[i * PD + f]) = vreg[u];
        }
        if (w == 0) {
            // within-chunk log decays (tokens past the end count as gamma = 1)
            float l = __logf(greg);
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
        if (c + 1 < n_chunks) prefetch(c + 1);

        // ---- the state before this chunk ----
        if (write_chunks) {
            float* dst = Sout + (size_t)c * D * D;
#pragma unroll
            for (int j = 0; j < NT; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    dst[(size_t)(m0 + 4 * kk + r) * D + 16 * j + n] = acc[j][r];
        }

        // ---- S <- Gamma_c S + sum_i w_i a_i k_i^T ----
        const float G = sGam;
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[j] *= G;
#pragma unroll
        for (int g = 0; g < C / 16; ++g) {
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int i = 16 * g + 4 * kk + s;
                const float a = sArows[i * PD + m0 + n] * sW[i];
#pragma unroll
                for (int j = 0; j < NT; ++j) acc[j] = mfma4(a, sK[i * PD + 16 * j + n], acc[j]);
            }
        }
        __syncthreads();
    }

    // ---- final state (after the last token) ----
    float* fin = which == 0 ? final_H : final_G;
    if (fin) {
        float* dst = fin + (size_t)bh * D * D;
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[(size_t)(m0 + 4 * kk + r) * D + 16 * j + n] = acc[j][r];
    }
}

template <int D, int C, typename In>
hipError_t launch_chunk_states_t(const ChunkStatesArgs& a, hipStream_t s) {
    constexpr int NW = D >= 64 ? 4 : D / 16;
    constexpr int RB = D / (16 * NW);
    // ids: 8 XCD lanes x (heads rounded up to a multiple of 8) / 8 x parts
    const long grid = ((a.BH + 7) / 8) * 8 * 2 * RB;
    hipLaunchKernelGGL((chunk_states_kernel<D, C, In>), dim3((unsigned)grid), dim3(64 * NW), 0, s,
                       (const In*)a.k, (const In*)a.v, a.gamma, a.T, a.n_chunks, a.SH, a.SG,
                       a.final_H, a.final_G, a.write_chunks, a.BH);
    return hipGetLastError();
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
