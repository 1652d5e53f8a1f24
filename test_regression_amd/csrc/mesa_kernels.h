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
    int* work_counter;   // zeroed for the CG kernel that follows, or nullptr
    int g_transposed;    // store G^T's blocks in operand order (the adjoint's A operand), not G's
};

struct CgOutputArgs {
    const void* q; const void* k; const void* v; const float* gamma; const float* lambda;
    const float* SH; const float* SG;
    long BH; int H; int T; int d; int chunk; int n_chunks; int bf16;
    int max_iters; float tol;
    float* out; int32_t* iters;
    float* x_out;   // CG solutions [BH, T, d], or nullptr
    int* work_counter;   // chunk claims; zero at launch
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

// Backward pass (see the bwd_*.hip kernels).
struct BwdAdjointArgs {
    const void* k; const void* v; const float* gamma; const float* lambda;
    const float* x; const float* o; const float* gout; const float* SH; const float* SG;
    long BH; int H; int T; int d; int chunk; int n_chunks; int bf16; int max_iters; float tol;
    float* dq; float* beta; int32_t* z_iters;
    float* lam_part;     // per chunk and wave: sum over the wave's tokens of z (.) x  [BH*n_chunks][C/16][d]
    int* work_counter;   // chunk claims; zero at launch
};
struct BwdStatesArgs {
    const float* g; const float* z; const float* x; const float* gamma;
    long BH; int T; int d; int chunk; int n_chunks;
    float* Pgx; float* Pzx;
    int* Egx; int* Ezx;   // d >= 32: the states' exponents per (head, chunk, row block)
};
struct BwdKvArgs {
    const void* k; const void* v; const float* gamma; const float* x; const float* z; const float* gout;
    const float* Pgx; const float* Pzx;
    const int* Egx; const int* Ezx;
    long BH; int T; int d; int chunk; int n_chunks; int bf16;
    float* dk; float* dv; float* akey;
};
struct BwdGateArgs {
    const float* beta; const float* akey; const float* gamma; const float* lam_part;
    long BH; int B; int H; int T; int d;
    int n_chunks;   // rows of lam_part per (batch, head): chunks times partial sums per chunk
    float* dgamma; float* dlam;
};

hipError_t launch_bwd_adjoint(const BwdAdjointArgs& a, hipStream_t s);
hipError_t launch_bwd_states(const BwdStatesArgs& a, hipStream_t s);
hipError_t launch_bwd_kv(const BwdKvArgs& a, hipStream_t s);
hipError_t launch_bwd_gate(const BwdGateArgs& a, hipStream_t s);
// Hawk layer recurrence (hawk.hip): two-pass chunked scan.
#ifndef MESA_HAWK_CHUNK
#define MESA_HAWK_CHUNK 128
#endif
constexpr int kHawkChunk = MESA_HAWK_CHUNK;   // tokens per chunk of the scan
struct HawkArgs {
    const void* x; const void* ga; const void* gx; const float* lam; float c; const float* h0;
    int B; int T; int D; int nc; int bf16;
    float* Plog; float* S;   // workspace: per (sequence, chunk, channel) log decay product, end state
    float* y; float* h_final;
};
hipError_t launch_hawk(const HawkArgs& a, hipStream_t s);

hipError_t launch_cg_output(const CgOutputArgs& a, hipStream_t s);
hipError_t launch_cg_output_bf16(const CgOutputArgs& a, hipStream_t s);   // bf16 q/k/v, d >= 32
hipError_t launch_qk_preprocess(const QkPreArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

}  // namespace mesa
