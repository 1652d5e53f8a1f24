// mesa_kernels.h -- host-side launch interface of the gfx950 Mesa-layer kernels.
// Internal to libmesa; the public ABI is include/mesa.h.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mesa {

struct ChunkStatesArgs {
    const void* k; const void* v; const float* gamma;
    long BH; int T; int d; int chunk; int n_chunks; int bf16;
    float* SH; float* SG; float* final_H; float* final_G; int write_chunks;
};

struct CgOutputArgs {
    const void* q; const void* k; const void* v; const float* gamma; const float* lambda;
    const float* SH; const float* SG;
    long BH; int H; int T; int d; int chunk; int n_chunks; int bf16;
    int max_iters; float tol;
    float* out; int32_t* iters;
};

struct DecodeArgs {
    const void* q; const void* k; const void* v; const float* gamma; const float* lambda;
    float* SH; float* SG;
    long NH; int H; int d; int bf16; int max_iters; float tol;
    float* out; int32_t* iters;
    float* X; int warm_mode;   // warm start: previous solutions [NH, d] (nullptr: cold)
};

hipError_t launch_chunk_states(const ChunkStatesArgs& a, hipStream_t s);
struct QkPreArgs {
    const void* x; const float* w; int W; const void* hist; void* hist_out;
    int H; int T;
    int segs_per_bh; long n_segs;   // token segments of the main kernel (B * H * segs_per_bh)
    long n_hist;                    // elements of hist_out (B * H * (W - 1) * d), when it is set
    int d; int in_bf16; int out_bf16;
    void* y;
};
#ifndef MESA_QK_PRE_SEGMENT
#define MESA_QK_PRE_SEGMENT 32
#endif
constexpr int kQkPreSegment = MESA_QK_PRE_SEGMENT;   // tokens per thread of the pre-processing kernel
constexpr int kQkPreMaxWidth = 4;   // widest convolution window the kernel is built for

hipError_t launch_cg_output(const CgOutputArgs& a, hipStream_t s);
hipError_t launch_qk_preprocess(const QkPreArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace mesa
