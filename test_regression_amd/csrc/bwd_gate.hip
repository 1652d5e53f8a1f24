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
// z (.) x).  Both sums run in double precision in a fixed order.
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

// dlambda[h][f] = -sum_{b, c} part[(b*H + h) * n_chunks + c][f]
__global__ __launch_bounds__(256) void bwd_lambda_kernel(const float* __restrict__ lam_part, int B, int H,
                                                         int n_chunks, int D, float* __restrict__ dlam) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i >= (long)H * D) return;
    const int h = (int)(i / D), f = (int)(i % D);
    double s = 0.0;
    for (int b = 0; b < B; ++b)
        for (int c = 0; c < n_chunks; ++c) s += lam_part[(((size_t)b * H + h) * n_chunks + c) * D + f];
    dlam[i] = (float)(-s);
}

hipError_t launch_bwd_gate(const BwdGateArgs& a, hipStream_t s) {
    if (a.T > 0) {
        hipLaunchKernelGGL(bwd_gate_kernel, dim3((unsigned)a.BH), dim3(256), 0, s, a.beta, a.akey, a.gamma, a.T,
                           a.dgamma);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    const long n = (long)a.H * a.d;
    hipLaunchKernelGGL(bwd_lambda_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, a.lam_part, a.B, a.H,
                       a.n_chunks, a.d, a.dlam);
    return hipGetLastError();
}

}  // namespace mesa
