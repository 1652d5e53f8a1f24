// bwd_gate.hip -- the backward's gate and regulariser gradients (gfx950).
//
// Implicit differentiation of o_t = G_t (H_t + Lambda)^{-1} q_t (the page,
// section "A Camada Mesa", bullet "Paralelizacao", says the layer trains in
// parallel but gives no gradient).  With zeta_ti = prod_{s=i+1..t} gamma_s,
// every pair i < s <= t carries ln gamma_s, so
//   dL/dln gamma_s = sum_{t >= s} (beta_t - a_t),
// beta_t the query-side and a_t the key-side per-token totals (computed by
// the adjoint and key/value kernels), and dL/dgamma_s = that / gamma_s.
// dL/dlambda = -(sum over the batch and chunks of the per-chunk sums of
// z (.) x).  Both sums run in double precision in an order fixed by the sizes.
#include "mesa_device.h"
#include "mesa_kernels.h"

namespace mesa {

// One workgroup per head: a reverse inclusive scan of (beta - a) over T.
__global__ __launch_bounds__(256) void bwd_gate_kernel(const float* __restrict__ beta,
                                                       const float* __restrict__ akey,
                                                       const float* __restrict__ gamma, int T,
                                                       float* __restrict__ dgamma) {
    __shared__ double part[256];
    const int tid = threadIdx.x;
    const size_t base = (size_t)blockIdx.x * T;
    const int per = (T + 255) / 256;
    const int lo = min(T, tid * per), hi = min(T, lo + per);
    double s = 0.0;
    for (int t = lo; t < hi; ++t) s += (double)beta[base + t] - (double)akey[base + t];
    part[tid] = s;
    __syncthreads();
    // suffix sums of the segment totals: part[i] <- sum_{j >= i} part[j]
    for (int o = 1; o < 256; o <<= 1) {
        const double add = tid + o < 256 ? part[tid + o] : 0.0;
        __syncthreads();
        part[tid] += add;
        __syncthreads();
    }
    double acc = tid + 1 < 256 ? part[tid + 1] : 0.0;   // everything after this segment
    for (int t = hi - 1; t >= lo; --t) {
        acc += (double)beta[base + t] - (double)akey[base + t];
        dgamma[base + t] = (float)(acc / (double)gamma[base + t]);
    }
}

// dlambda[h][f] = -sum_{b, c} part[(b*H + h) * n_chunks + c][f].  One
// 1024-thread workgroup per (head, 64 features): a thread takes 4 features
// (one 16-byte load per row) and the rows congruent to its row group mod 64,
// in order; then the 64 partial sums are added in order.  The order is
// fixed by the sizes alone.
constexpr int kLamGroups = 64;
__global__ __launch_bounds__(1024) void bwd_lambda_kernel(const float* __restrict__ lam_part, int B, int H,
                                                          int n_chunks, int D, float* __restrict__ dlam) {
    __shared__ double part[kLamGroups][64];
    const int q = threadIdx.x & 15, r = threadIdx.x >> 4;   // feature quad, row group
    const int fblocks = (D + 63) / 64;
    const int h = blockIdx.x / fblocks;
    const int f0 = (blockIdx.x % fblocks) * 64 + 4 * q;
    const long rows = (long)B * n_chunks;
    double s0 = 0.0, s1 = 0.0, s2 = 0.0, s3 = 0.0;
    if (f0 < D) {   // D is a multiple of 16, so the quad is whole
        for (long j = r; j < rows; j += kLamGroups) {
            const long b = j / n_chunks, c = j % n_chunks;
            const f32x4 v = *reinterpret_cast<const f32x4*>(lam_part + (((size_t)b * H + h) * n_chunks + c) * D + f0);
            s0 += v[0];
            s1 += v[1];
            s2 += v[2];
            s3 += v[3];
        }
    }
    part[r][4 * q] = s0;
    part[r][4 * q + 1] = s1;
    part[r][4 * q + 2] = s2;
    part[r][4 * q + 3] = s3;
    __syncthreads();
    const int f = (blockIdx.x % fblocks) * 64 + threadIdx.x;
    if (threadIdx.x < 64 && f < D) {
        double t = 0.0;
        for (int g = 0; g < kLamGroups; ++g) t += part[g][threadIdx.x];
        dlam[(size_t)h * D + f] = (float)(-t);
    }
}

hipError_t launch_bwd_gate(const BwdGateArgs& a, hipStream_t s) {
    if (a.T > 0) {
        hipLaunchKernelGGL(bwd_gate_kernel, dim3((unsigned)a.BH), dim3(256), 0, s, a.beta, a.akey, a.gamma, a.T,
                           a.dgamma);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long blocks = (long)a.H * ((a.d + 63) / 64);
    hipLaunchKernelGGL(bwd_lambda_kernel, dim3((unsigned)blocks), dim3(1024), 0, s, a.lam_part, a.B, a.H,
                       a.n_chunks, a.d, a.dlam);
    return hipGetLastError();
}

}  // namespace mesa
