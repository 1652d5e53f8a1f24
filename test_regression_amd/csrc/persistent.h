// persistent.h -- chunk bookkeeping of the persistent chunk kernels (gfx950).
//
// The CG kernels of the forward and of the backward's adjoint solve run as
// many workgroups as are resident at once; each starts on chunk blockIdx.x
// and then claims chunks in order from a counter in the workspace, so that
// chunks whose CG runs longer do not hold up a fixed share of the work.
#pragma once
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>

namespace mesa {

// Where a chunk lives in the inputs and the workspace.
struct ChunkPos {
    size_t tok0;   // first token of the chunk (row of the [B*H*T, d] inputs)
    size_t hoff;   // offset of its packed S^H_c
    size_t soff;   // offset of its S^G_c
    int h;         // head
    int valid;     // tokens of the chunk inside the sequence
};

template <int D, int C>
__device__ __forceinline__ ChunkPos chunk_pos(long idx, int n_chunks, int H, int T) {
    constexpr int HPACK = D * (D + 16) / 2;   // packed upper block triangle of S^H
    ChunkPos p;
    const int c = (int)(idx % n_chunks);
    const long bh = idx / n_chunks;
    p.h = (int)(bh % H);
    p.valid = min(C, T - c * C);
    p.tok0 = (size_t)bh * T + (size_t)c * C;
    p.hoff = (size_t)idx * HPACK;
    p.soff = (size_t)idx * D * D;
    return p;
}

constexpr int kMaxDevices = 64;

// Workgroups of `kernel` resident at once on the current device (cached per device).
template <typename Kernel>
static long resident_workgroups(Kernel kernel, int block, std::atomic<long> (&cache)[kMaxDevices]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    long r = cache[dev].load(std::memory_order_relaxed);
    if (r > 0) return r;
    int cus = 0, per = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, kernel, block, 0) != hipSuccess || per < 1) per = 1;
    r = (long)cus * per;
    cache[dev].store(r, std::memory_order_relaxed);
    return r;
}

}  // namespace mesa
