// mesa_host.hip -- the C ABI of libmesa (declared in include/mesa.h).
//
// Host-side only: validates every argument before anything is enqueued,
// carves the caller's workspace, and enqueues the kernels on the caller's
// stream.  Allocates no device memory and never synchronises (except in
// mesa_profile_read, which waits for its own events).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/mesa.h"
#include "mesa_kernels.h"

namespace {

thread_local std::string g_err;

mesa_status fail(mesa_status s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return s;
}

mesa_status hip_fail(hipError_t e, const char* what) {
    return fail(MESA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_d(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }

constexpr int kMaxIters = 4096;

// ---------------- optional per-kernel timing ----------------
struct ProfRec { hipEvent_t a, b; int kid; };
std::mutex g_prof_mu;
bool g_prof_on = false;
std::vector<ProfRec> g_prof_pending;
double g_prof_ms[MESA_KERNEL_COUNT] = {};
int64_t g_prof_n[MESA_KERNEL_COUNT] = {};

// Launches `fn` on `s`; when profiling is on (and `may_record`), brackets it
// with two events.
template <typename Fn>
hipError_t timed_launch(int kid, hipStream_t s, Fn fn, bool may_record = true) {
    bool on;
    {
        std::lock_guard<std::mutex> g(g_prof_mu);
        on = g_prof_on && may_record;
    }
    if (!on) return fn();
    ProfRec r{nullptr, nullptr, kid};
    hipError_t e = hipEventCreate(&r.a);
    if (e != hipSuccess) return e;
    e = hipEventCreate(&r.b);
    if (e == hipSuccess) e = hipEventRecord(r.a, s);
    if (e == hipSuccess) e = fn();
    if (e == hipSuccess) e = hipEventRecord(r.b, s);
    if (e != hipSuccess) {
        (void)hipEventDestroy(r.a);
        if (r.b) (void)hipEventDestroy(r.b);
        return e;
    }
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_pending.push_back(r);
    return hipSuccess;
}

// Zero-fill with a kernel rather than hipMemsetAsync, so that a caller may
// capture the call in a HIP graph.
__global__ void zero_fill_kernel(uint32_t* p, size_t n_words) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_words;
         i += (size_t)gridDim.x * blockDim.x)
        p[i] = 0u;
}

hipError_t zero_fill(void* p, size_t bytes, hipStream_t s) {
    if (!p || bytes == 0) return hipSuccess;
    const size_t words = bytes / 4;   // every buffer filled here is 4-byte elements
    const unsigned blocks = (unsigned)std::min<size_t>((words + 255) / 256, 4096);
    hipLaunchKernelGGL(zero_fill_kernel, dim3(blocks), dim3(256), 0, s, static_cast<uint32_t*>(p), words);
    return hipGetLastError();
}

}  // namespace

extern "C" {

int mesa_abi_version(void) { return MESA_ABI_VERSION; }

const char* mesa_status_string(int s) {
    switch (s) {
        case MESA_OK: return "MESA_OK";
        case MESA_ERR_INVALID_ARGUMENT: return "MESA_ERR_INVALID_ARGUMENT";
        case MESA_ERR_UNSUPPORTED: return "MESA_ERR_UNSUPPORTED";
        case MESA_ERR_WORKSPACE_TOO_SMALL: return "MESA_ERR_WORKSPACE_TOO_SMALL";
        case MESA_ERR_HIP: return "MESA_ERR_HIP";
    }
    return "MESA_ERR_UNKNOWN";
}

const char* mesa_last_error_message(void) { return g_err.c_str(); }

// Bytes of the forward's chunk states: per chunk and head the packed upper
// 16x16-block triangle of H (dk (dk + 16) / 2 floats) and the full G
// (dv x dk), fp32.  A 256-byte tail after them holds the CG/output kernel's
// chunk-claim counter.
static size_t forward_state_bytes(long BH, long nc, int dk, int dv) {
    return (size_t)BH * nc * ((size_t)dk * (dk + 16) / 2 + (size_t)dv * dk) * sizeof(float);
}
constexpr size_t kForwardTailBytes = 256;

size_t mesa_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
    const long nc = ((long)T + chunk - 1) / chunk;
    if (nc == 0) return 0;
    return forward_state_bytes((long)B * H, nc, dk, dv) + kForwardTailBytes;
}

static mesa_status forward_impl(const void* q, const void* k, const void* v, int qkv_dtype,
                                const float* gamma, const float* lambda, int B, int H, int T, int dk,
                                int dv, int chunk, int max_iters, float tol, float* out, int32_t* iters,
                                float* final_H, float* final_G, float* x_out, void* workspace,
                                size_t workspace_bytes, void* stream, bool may_record = true) {
    if (qkv_dtype != MESA_DTYPE_F32 && qkv_dtype != MESA_DTYPE_BF16)
        return fail(MESA_ERR_INVALID_ARGUMENT, "qkv_dtype %d is not MESA_DTYPE_F32 or MESA_DTYPE_BF16", qkv_dtype);
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || chunk <= 0)
        return fail(MESA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d H=%d T=%d dk=%d dv=%d chunk=%d)",
                    B, H, T, dk, dv, chunk);
    if (max_iters < 0 || max_iters > kMaxIters)
        return fail(MESA_ERR_INVALID_ARGUMENT, "max_iters=%d outside [0, %d]", max_iters, kMaxIters);
    if (!(tol >= 0.0f) || std::isinf(tol))
        return fail(MESA_ERR_INVALID_ARGUMENT, "tol must be finite and >= 0");
    const bool need_ws = max_iters > 0 && T > 0;
    if (T > 0 && (!q || !k || !v || !gamma || !out))
        return fail(MESA_ERR_INVALID_ARGUMENT, "q, k, v, gamma and out must be non-null");
    if (!lambda) return fail(MESA_ERR_INVALID_ARGUMENT, "lambda must be non-null");
    if (need_ws && !workspace) return fail(MESA_ERR_INVALID_ARGUMENT, "workspace must be non-null when max_iters > 0");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(final_H, 16) || !aligned(final_G, 16) || !aligned(workspace, 16) || !aligned(x_out, 16) ||
        !aligned(gamma, 4) || !aligned(lambda, 4) || !aligned(iters, 4))
        return fail(MESA_ERR_INVALID_ARGUMENT, "misaligned pointer (16 B for tensors/workspace, 4 B for gamma/lambda/iters)");
    if (dk != dv) return fail(MESA_ERR_UNSUPPORTED, "dk (%d) != dv (%d) is not built", dk, dv);
    if (!supported_d(dk)) return fail(MESA_ERR_UNSUPPORTED, "d=%d not built (16, 32, 64, 128)", dk);
    if (!supported_chunk(chunk)) return fail(MESA_ERR_UNSUPPORTED, "chunk=%d not built (16, 32, 64)", chunk);
    const long n_chunks = ((long)T + chunk - 1) / chunk;
    const long BH = (long)B * H;
    if (BH * 4 > 0x7fffffffL || BH * n_chunks > 0x7fffffffL)
        return fail(MESA_ERR_INVALID_ARGUMENT, "grid too large (B*H=%ld, chunks=%ld)", BH, n_chunks);
    if (need_ws) {
        const size_t need = mesa_forward_workspace_bytes(B, H, T, dk, dv, chunk);
        if (workspace_bytes < need)
            return fail(MESA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    }
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int bf16 = qkv_dtype == MESA_DTYPE_BF16;
    float* SH = static_cast<float*>(workspace);
    float* SG = need_ws ? SH + (size_t)BH * n_chunks * ((size_t)dk * (dk + 16) / 2) : nullptr;
    int* work_counter =
        need_ws ? reinterpret_cast<int*>(static_cast<char*>(workspace) + forward_state_bytes(BH, n_chunks, dk, dv))
                : nullptr;

    if (T == 0) {
        // Nothing to solve; the final states are the zero initial states.
        hipError_t e = zero_fill(final_H, (size_t)BH * dk * dk * sizeof(float), s);
        if (e == hipSuccess) e = zero_fill(final_G, (size_t)BH * dv * dk * sizeof(float), s);
        if (e != hipSuccess) return hip_fail(e, "zero fill of the final states");
        return MESA_OK;
    }

    if (need_ws || final_H || final_G) {
        mesa::ChunkStatesArgs a{k, v, gamma, BH, T, dk, chunk, (int)n_chunks, bf16,
                                SH, SG, final_H, final_G, need_ws ? 1 : 0, work_counter, 0};
        hipError_t e = timed_launch(
            MESA_KERNEL_CHUNK_STATES, s, [&] { return mesa::launch_chunk_states(a, s); }, may_record);
        if (e != hipSuccess) return hip_fail(e, "chunk-state kernel launch");
    }
    if (!need_ws) {
        // max_iters == 0: x = 0, so out = 0 and no update is made.
        hipError_t e = zero_fill(out, (size_t)BH * T * dv * sizeof(float), s);
        if (e == hipSuccess) e = zero_fill(iters, (size_t)BH * T * sizeof(int32_t), s);
        if (e == hipSuccess) e = zero_fill(x_out, (size_t)BH * T * dk * sizeof(float), s);
        if (e != hipSuccess) return hip_fail(e, "zero fill of out/iters");
        return MESA_OK;
    }
    mesa::CgOutputArgs a{q, k, v, gamma, lambda, SH, SG, BH, H, T, dk, chunk, (int)n_chunks,
                         bf16, max_iters, tol, out, iters, x_out, work_counter};
    hipError_t e =
        timed_launch(MESA_KERNEL_CG_OUTPUT, s, [&] { return mesa::launch_cg_output(a, s); }, may_record);
    if (e != hipSuccess) return hip_fail(e, "CG/output kernel launch");
    return MESA_OK;
}

mesa_status mesa_forward(const void* q, const void* k, const void* v, int qkv_dtype,
                         const float* gamma, const float* lambda, int B, int H, int T, int dk,
                         int dv, int chunk, int max_iters, float tol, float* out, int32_t* iters,
                         float* final_H, float* final_G, void* workspace, size_t workspace_bytes,
                         void* stream) {
    g_err.clear();
    return forward_impl(q, k, v, qkv_dtype, gamma, lambda, B, H, T, dk, dv, chunk, max_iters, tol, out, iters,
                        final_H, final_G, nullptr, workspace, workspace_bytes, stream);
}

mesa_status mesa_forward_train(const void* q, const void* k, const void* v, int qkv_dtype,
                               const float* gamma, const float* lambda, int B, int H, int T, int dk,
                               int dv, int chunk, int max_iters, float tol, float* out, int32_t* iters,
                               float* x_out, void* workspace, size_t workspace_bytes, void* stream) {
    g_err.clear();
    if (T > 0 && !x_out) return fail(MESA_ERR_INVALID_ARGUMENT, "x_out must be non-null");
    return forward_impl(q, k, v, qkv_dtype, gamma, lambda, B, H, T, dk, dv, chunk, max_iters, tol, out, iters,
                        nullptr, nullptr, x_out, workspace, workspace_bytes, stream);
}

}  // extern "C"

// ---- the forward without a caller workspace ----
// The chunk states and the claim counter live in this file-scope device
// array instead.  Each GPU the library runs on holds its own copy until the
// process ends; in host code the name only stands for the array, so the
// library reads each device's address once (with that device current) and
// passes that address to the kernels.
static __device__ __align__(256) unsigned char scratch[MESA_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
constexpr int kScratchDevices = 64;
void* g_scratch_ptr[kScratchDevices] = {};

mesa_status scratch_of_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kScratchDevices)
        return fail(MESA_ERR_UNSUPPORTED, "device %d beyond the %d this build tracks", dev, kScratchDevices);
    std::lock_guard<std::mutex> g(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress of the scratch array");
        if (!p) return fail(MESA_ERR_HIP, "hipGetSymbolAddress gave a null scratch address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return MESA_OK;
}
}  // namespace

extern "C" {

mesa_status mesa_forward_noalloc(const void* q, const void* k, const void* v, int qkv_dtype,
                                 const float* gamma, const float* lambda, int B, int H, int T, int dk,
                                 int dv, int chunk, int max_iters, float tol, float* out, int32_t* iters,
                                 float* final_H, float* final_G, void* stream) {
    g_err.clear();
    void* ws = nullptr;
    size_t ws_bytes = 0;
    if (max_iters > 0 && T > 0) {
        ws_bytes = mesa_forward_workspace_bytes(B, H, T, dk, dv, chunk);
        if (ws_bytes > MESA_NOALLOC_SCRATCH_BYTES)
            return fail(MESA_ERR_WORKSPACE_TOO_SMALL,
                        "these sizes need %zu bytes of chunk states; the built-in scratch holds %zu "
                        "(use mesa_forward with a caller workspace)",
                        ws_bytes, (size_t)MESA_NOALLOC_SCRATCH_BYTES);
        if (ws_bytes > 0) {
            const mesa_status st = scratch_of_current_device(&ws);
            if (st != MESA_OK) return st;
        }
    }
    return forward_impl(q, k, v, qkv_dtype, gamma, lambda, B, H, T, dk, dv, chunk, max_iters, tol, out, iters,
                        final_H, final_G, nullptr, ws, ws_bytes, stream, /*may_record=*/false);
}

// Backward workspace: forward chunk states, reverse states, per-token totals,
// per-chunk regulariser sums; every segment a multiple of 4 floats.
struct BwdLayout {
    size_t sh, sg, pgx, pzx, egx, ezx, beta, akey, lam, counter, total;   // offsets in floats
};

// lam: one d-vector per chunk and 16-token wave of the adjoint kernel;
// counter: the adjoint kernel's chunk-claim counter (64 floats = 256 bytes).
static BwdLayout bwd_layout(long BH, int T, int d, long nc, int chunk) {
    auto r4 = [](size_t n) { return (n + 3) / 4 * 4; };
    const size_t waves = (size_t)std::max(1, chunk / 16);
    BwdLayout l{};
    size_t o = 0;
    l.sh = o;   o += r4((size_t)BH * nc * ((size_t)d * (d + 16) / 2));
    l.sg = o;   o += r4((size_t)BH * nc * d * d);
    l.pgx = o;  o += r4((size_t)BH * nc * d * d);   // P^gx, accumulator block order
    l.pzx = o;  o += r4((size_t)BH * nc * d * d);   // P^zx + (P^zx)^T, accumulator block order
    l.egx = o;  o += r4((size_t)BH * nc * (d / 16));   // their exponents per 16-row block (d >= 32)
    l.ezx = o;  o += r4((size_t)BH * nc * (d / 16));
    l.beta = o; o += r4((size_t)BH * T);
    l.akey = o; o += r4((size_t)BH * T);
    l.lam = o;  o += r4((size_t)BH * nc * waves * d);
    l.counter = o; o += 64;
    l.total = o;
    return l;
}

size_t mesa_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk) {
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || chunk <= 0) return 0;
    const long nc = ((long)T + chunk - 1) / chunk;
    return bwd_layout((long)B * H, T, std::max(dk, dv), nc, chunk).total * sizeof(float);
}

mesa_status mesa_backward(const void* k, const void* v, int qkv_dtype, const float* gamma, const float* lambda,
                          const float* x, const float* out, const float* grad_out, int B, int H, int T, int dk,
                          int dv, int chunk, int max_iters, float tol, float* grad_q, float* grad_k, float* grad_v,
                          float* grad_gamma, float* grad_lambda, int32_t* z_iters, void* workspace,
                          size_t workspace_bytes, void* stream) {
    g_err.clear();
    if (qkv_dtype != MESA_DTYPE_F32 && qkv_dtype != MESA_DTYPE_BF16)
        return fail(MESA_ERR_INVALID_ARGUMENT, "qkv_dtype %d is not MESA_DTYPE_F32 or MESA_DTYPE_BF16", qkv_dtype);
    if (B <= 0 || H <= 0 || T < 0 || dk <= 0 || dv <= 0 || chunk <= 0)
        return fail(MESA_ERR_INVALID_ARGUMENT, "sizes must be positive (B=%d H=%d T=%d dk=%d dv=%d chunk=%d)",
                    B, H, T, dk, dv, chunk);
    if (max_iters < 0 || max_iters > kMaxIters)
        return fail(MESA_ERR_INVALID_ARGUMENT, "max_iters=%d outside [0, %d]", max_iters, kMaxIters);
    if (!(tol >= 0.0f) || std::isinf(tol))
        return fail(MESA_ERR_INVALID_ARGUMENT, "tol must be finite and >= 0");
    if (!lambda || !grad_lambda) return fail(MESA_ERR_INVALID_ARGUMENT, "lambda and grad_lambda must be non-null");
    if (T > 0 && (!k || !v || !gamma || !x || !out || !grad_out || !grad_q || !grad_k || !grad_v || !grad_gamma))
        return fail(MESA_ERR_INVALID_ARGUMENT, "k, v, gamma, x, out, grad_out and the gradients must be non-null");
    if (T > 0 && !workspace) return fail(MESA_ERR_INVALID_ARGUMENT, "workspace must be non-null");
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(x, 16) || !aligned(out, 16) || !aligned(grad_out, 16) ||
        !aligned(grad_q, 16) || !aligned(grad_k, 16) || !aligned(grad_v, 16) || !aligned(workspace, 16) ||
        !aligned(gamma, 4) || !aligned(lambda, 4) || !aligned(grad_gamma, 4) || !aligned(grad_lambda, 4) ||
        !aligned(z_iters, 4))
        return fail(MESA_ERR_INVALID_ARGUMENT, "misaligned pointer (16 B for tensors/workspace, 4 B for the rest)");
    if (dk != dv) return fail(MESA_ERR_UNSUPPORTED, "dk (%d) != dv (%d) is not built", dk, dv);
    if (!supported_d(dk)) return fail(MESA_ERR_UNSUPPORTED, "d=%d not built (16, 32, 64, 128)", dk);
    if (!supported_chunk(chunk)) return fail(MESA_ERR_UNSUPPORTED, "chunk=%d not built (16, 32, 64)", chunk);
    const long n_chunks = ((long)T + chunk - 1) / chunk;
    const long BH = (long)B * H;
    if (BH * 4 > 0x7fffffffL || BH * n_chunks > 0x7fffffffL)
        return fail(MESA_ERR_INVALID_ARGUMENT, "grid too large (B*H=%ld, chunks=%ld)", BH, n_chunks);
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        hipError_t e = zero_fill(grad_lambda, (size_t)H * dk * sizeof(float), s);
        if (e != hipSuccess) return hip_fail(e, "zero fill of grad_lambda");
        return MESA_OK;
    }
    const BwdLayout lay = bwd_layout(BH, T, dk, n_chunks, chunk);
    const int waves = chunk / 16;   // per-wave partial sums of z (.) x per chunk
    if (workspace_bytes < lay.total * sizeof(float))
        return fail(MESA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes,
                    lay.total * sizeof(float));
    float* ws = static_cast<float*>(workspace);
    const int bf16 = qkv_dtype == MESA_DTYPE_BF16;
    hipError_t e;
    {
        mesa::ChunkStatesArgs a{k, v, gamma, BH, T, dk, chunk, (int)n_chunks, bf16,
                                ws + lay.sh, ws + lay.sg, nullptr, nullptr, 1,
                                reinterpret_cast<int*>(ws + lay.counter), 1};
        e = timed_launch(MESA_KERNEL_CHUNK_STATES, s, [&] { return mesa::launch_chunk_states(a, s); });
        if (e != hipSuccess) return hip_fail(e, "chunk-state kernel launch");
    }
    {
        mesa::BwdAdjointArgs a{k, v, gamma, lambda, x, out, grad_out, ws + lay.sh, ws + lay.sg, BH, H, T, dk, chunk,
                               (int)n_chunks, bf16, max_iters, tol, grad_q, ws + lay.beta, z_iters, ws + lay.lam,
                               reinterpret_cast<int*>(ws + lay.counter)};
        e = timed_launch(MESA_KERNEL_BWD_ADJOINT, s, [&] { return mesa::launch_bwd_adjoint(a, s); });
        if (e != hipSuccess) return hip_fail(e, "backward adjoint kernel launch");
    }
    {
        mesa::BwdStatesArgs a{grad_out, grad_q, x, gamma, BH, T, dk, chunk, (int)n_chunks, ws + lay.pgx,
                              ws + lay.pzx, reinterpret_cast<int*>(ws + lay.egx),
                              reinterpret_cast<int*>(ws + lay.ezx)};
        e = timed_launch(MESA_KERNEL_BWD_STATES, s, [&] { return mesa::launch_bwd_states(a, s); });
        if (e != hipSuccess) return hip_fail(e, "backward state kernel launch");
    }
    {
        mesa::BwdKvArgs a{k, v, gamma, x, grad_q, grad_out, ws + lay.pgx, ws + lay.pzx,
                          reinterpret_cast<const int*>(ws + lay.egx), reinterpret_cast<const int*>(ws + lay.ezx),
                          BH, T, dk, chunk,
                          (int)n_chunks, bf16, grad_k, grad_v, ws + lay.akey};
        e = timed_launch(MESA_KERNEL_BWD_KV, s, [&] { return mesa::launch_bwd_kv(a, s); });
        if (e != hipSuccess) return hip_fail(e, "backward key/value kernel launch");
    }
    {
        mesa::BwdGateArgs a{ws + lay.beta, ws + lay.akey, gamma, ws + lay.lam, BH, B, H, T, dk,
                            (int)n_chunks * waves, grad_gamma, grad_lambda};
        e = timed_launch(MESA_KERNEL_BWD_GATE, s, [&] { return mesa::launch_bwd_gate(a, s); });
        if (e != hipSuccess) return hip_fail(e, "backward gate kernel launch");
    }
    return MESA_OK;
}

static mesa_status decode_impl(const char* what, const void* q, const void* k, const void* v, int qkv_dtype,
                               const float* gamma, const float* lambda, float* state_H, float* state_G,
                               float* state_x, int warm_mode, int N, int H, int dk, int dv, int max_iters,
                               float tol, float* out, int32_t* iters, void* stream) {
    g_err.clear();
    if (qkv_dtype != MESA_DTYPE_F32 && qkv_dtype != MESA_DTYPE_BF16)
        return fail(MESA_ERR_INVALID_ARGUMENT, "qkv_dtype %d is not MESA_DTYPE_F32 or MESA_DTYPE_BF16", qkv_dtype);
    if (N <= 0 || H <= 0 || dk <= 0 || dv <= 0)
        return fail(MESA_ERR_INVALID_ARGUMENT, "sizes must be positive (N=%d H=%d dk=%d dv=%d)", N, H, dk, dv);
    if (max_iters < 0 || max_iters > kMaxIters)
        return fail(MESA_ERR_INVALID_ARGUMENT, "max_iters=%d outside [0, %d]", max_iters, kMaxIters);
    if (!(tol >= 0.0f) || std::isinf(tol))
        return fail(MESA_ERR_INVALID_ARGUMENT, "tol must be finite and >= 0");
    if (!q || !k || !v || !gamma || !lambda || !state_H || !state_G || !out)
        return fail(MESA_ERR_INVALID_ARGUMENT, "q, k, v, gamma, lambda, state_H, state_G and out must be non-null");
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
        !aligned(state_H, 16) || !aligned(state_G, 16) || !aligned(gamma, 4) ||
        !aligned(lambda, 4) || !aligned(iters, 4) || !aligned(state_x, 16))
        return fail(MESA_ERR_INVALID_ARGUMENT, "misaligned pointer (16 B for tensors, 4 B for gamma/lambda/iters)");
    if (dk != dv) return fail(MESA_ERR_UNSUPPORTED, "dk (%d) != dv (%d) is not built", dk, dv);
    if (!supported_d(dk)) return fail(MESA_ERR_UNSUPPORTED, "d=%d not built (16, 32, 64, 128)", dk);
    const long NH = (long)N * H;
    if (NH > 0x7fffffffL) return fail(MESA_ERR_INVALID_ARGUMENT, "grid too large (N*H=%ld)", NH);
    hipStream_t s = static_cast<hipStream_t>(stream);
    mesa::DecodeArgs a{q, k, v, gamma, lambda, state_H, state_G, NH, H, dk,
                       qkv_dtype == MESA_DTYPE_BF16, max_iters, tol, out, iters, state_x, warm_mode};
    hipError_t e = timed_launch(MESA_KERNEL_DECODE, s, [&] { return mesa::launch_decode(a, s); });
    if (e != hipSuccess) return hip_fail(e, what);
    return MESA_OK;
}

mesa_status mesa_decode_step(const void* q, const void* k, const void* v, int qkv_dtype,
                             const float* gamma, const float* lambda, float* state_H,
                             float* state_G, int N, int H, int dk, int dv, int max_iters,
                             float tol, float* out, int32_t* iters, void* stream) {
    return decode_impl("decode kernel launch", q, k, v, qkv_dtype, gamma, lambda, state_H, state_G, nullptr, 0,
                       N, H, dk, dv, max_iters, tol, out, iters, stream);
}

mesa_status mesa_decode_step_warm(const void* q, const void* k, const void* v, int qkv_dtype,
                                  const float* gamma, const float* lambda, float* state_H,
                                  float* state_G, float* state_x, int N, int H, int dk, int dv,
                                  int max_iters, float tol, int warm_mode, float* out, int32_t* iters,
                                  void* stream) {
    g_err.clear();
    if (!state_x) return fail(MESA_ERR_INVALID_ARGUMENT, "state_x must be non-null");
    if (warm_mode != MESA_WARM_COLD && warm_mode != MESA_WARM_PREVIOUS && warm_mode != MESA_WARM_PROJECTED)
        return fail(MESA_ERR_INVALID_ARGUMENT, "warm_mode %d is not MESA_WARM_COLD, MESA_WARM_PREVIOUS or "
                    "MESA_WARM_PROJECTED", warm_mode);
    return decode_impl("warm decode kernel launch", q, k, v, qkv_dtype, gamma, lambda, state_H, state_G, state_x,
                       warm_mode, N, H, dk, dv, max_iters, tol, out, iters, stream);
}

mesa_status mesa_qk_preprocess(const void* x, int in_dtype, const float* conv_w, int width, const void* hist,
                               void* hist_out, int B, int H, int T, int d, void* y, int out_dtype,
                               void* stream) {
    g_err.clear();
    auto dtype_ok = [](int t) { return t == MESA_DTYPE_F32 || t == MESA_DTYPE_BF16; };
    if (!dtype_ok(in_dtype) || !dtype_ok(out_dtype))
        return fail(MESA_ERR_INVALID_ARGUMENT, "in_dtype %d / out_dtype %d must be MESA_DTYPE_F32 or "
                    "MESA_DTYPE_BF16", in_dtype, out_dtype);
    if (B <= 0 || H <= 0 || T < 0 || d <= 0)
        return fail(MESA_ERR_INVALID_ARGUMENT, "sizes must be positive, T >= 0 (B=%d H=%d T=%d d=%d)", B, H, T, d);
    if (width < 1 || width > 8) return fail(MESA_ERR_INVALID_ARGUMENT, "width=%d outside [1, 8]", width);
    if (!conv_w || (T > 0 && (!x || !y)))
        return fail(MESA_ERR_INVALID_ARGUMENT, "conv_w, and x and y when T > 0, must be non-null");
    if (!aligned(x, 16) || !aligned(y, 16) || !aligned(hist, 16) || !aligned(hist_out, 16) ||
        !aligned(conv_w, 16))
        return fail(MESA_ERR_INVALID_ARGUMENT, "misaligned pointer (16 B for every tensor)");
    if (y && y == x) return fail(MESA_ERR_INVALID_ARGUMENT, "y must not alias x");
    if (hist_out && (hist_out == hist || hist_out == x))
        return fail(MESA_ERR_INVALID_ARGUMENT, "hist_out must not alias hist or x");
    if (!supported_d(d)) return fail(MESA_ERR_UNSUPPORTED, "d=%d not built (16, 32, 64, 128)", d);
    if (width > mesa::kQkPreMaxWidth)
        return fail(MESA_ERR_UNSUPPORTED, "width=%d not built (at most %d)", width, mesa::kQkPreMaxWidth);
    const int segs = (T + mesa::kQkPreSegment - 1) / mesa::kQkPreSegment;
    const long n_segs = (long)B * H * segs;
    const long n_hist = (width > 1 && hist_out) ? (long)B * H * (width - 1) * d : 0;
    if (n_segs * d > 0x7fffffffL * 256L || n_hist > 0x7fffffffL * 256L)
        return fail(MESA_ERR_INVALID_ARGUMENT, "grid too large (B*H=%ld)", (long)B * H);
    if (n_segs == 0 && n_hist == 0) return MESA_OK;
    hipStream_t s = static_cast<hipStream_t>(stream);
    mesa::QkPreArgs a{x, conv_w, width, hist, n_hist ? hist_out : nullptr, H, T, segs, n_segs, n_hist, d,
                      in_dtype == MESA_DTYPE_BF16, out_dtype == MESA_DTYPE_BF16, y};
    hipError_t e = timed_launch(MESA_KERNEL_QK_PREPROCESS, s, [&] { return mesa::launch_qk_preprocess(a, s); });
    if (e != hipSuccess) return hip_fail(e, "q/k pre-processing kernel launch");
    return MESA_OK;
}

size_t mesa_hawk_workspace_bytes(int B, int T, int D) {
    if (B <= 0 || T < 0 || D <= 0) return 0;
    const size_t nc = ((size_t)T + mesa::kHawkChunk - 1) / mesa::kHawkChunk;
    return 2 * (size_t)B * nc * D * sizeof(float);
}

mesa_status mesa_hawk_scan(const void* x, const void* ga, const void* gx, int in_dtype, const float* lam, float c,
                           const float* h0, int B, int T, int D, float* y, float* h_final, void* workspace,
                           size_t workspace_bytes, void* stream) {
    g_err.clear();
    if (in_dtype != MESA_DTYPE_F32 && in_dtype != MESA_DTYPE_BF16)
        return fail(MESA_ERR_INVALID_ARGUMENT, "in_dtype %d is not MESA_DTYPE_F32 or MESA_DTYPE_BF16", in_dtype);
    if (B <= 0 || T < 0 || D <= 0)
        return fail(MESA_ERR_INVALID_ARGUMENT, "sizes must be positive, T >= 0 (B=%d T=%d D=%d)", B, T, D);
    if (!(c >= 0.0f) || std::isinf(c)) return fail(MESA_ERR_INVALID_ARGUMENT, "c must be finite and >= 0");
    if (!lam || (T > 0 && (!x || !ga || !gx || !y || !workspace)))
        return fail(MESA_ERR_INVALID_ARGUMENT, "lam, and x, ga, gx, y and workspace when T > 0, must be non-null");
    const size_t esz = in_dtype == MESA_DTYPE_BF16 ? 2 : 4;
    if (!aligned(x, esz) || !aligned(ga, esz) || !aligned(gx, esz) || !aligned(lam, 4) || !aligned(h0, 4) ||
        !aligned(y, 4) || !aligned(h_final, 4) || !aligned(workspace, 16))
        return fail(MESA_ERR_INVALID_ARGUMENT, "misaligned pointer");
    if (y && (y == x || y == ga || y == gx)) return fail(MESA_ERR_INVALID_ARGUMENT, "y must not alias the inputs");
    const long nc = ((long)T + mesa::kHawkChunk - 1) / mesa::kHawkChunk;
    if ((long)B * nc * D > 0x7fffffffL * 256L) return fail(MESA_ERR_INVALID_ARGUMENT, "grid too large");
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (T == 0) {
        // no token: the final state is the initial one
        hipError_t e = hipSuccess;
        if (h_final) {
            e = h0 ? hipMemcpyAsync(h_final, h0, (size_t)B * D * sizeof(float), hipMemcpyDeviceToDevice, s)
                   : zero_fill(h_final, (size_t)B * D * sizeof(float), s);
        }
        if (e != hipSuccess) return hip_fail(e, "Hawk final state for T = 0");
        return MESA_OK;
    }
    if (workspace_bytes < mesa_hawk_workspace_bytes(B, T, D))
        return fail(MESA_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", workspace_bytes,
                    mesa_hawk_workspace_bytes(B, T, D));
    float* ws = static_cast<float*>(workspace);
    const size_t per = (size_t)B * nc * D;
    mesa::HawkArgs a{x, ga, gx, lam, c, h0, B, T, D, (int)nc, in_dtype == MESA_DTYPE_BF16, ws, ws + per, y,
                     h_final};
    hipError_t e = timed_launch(MESA_KERNEL_HAWK, s, [&] { return mesa::launch_hawk(a, s); });
    if (e != hipSuccess) return hip_fail(e, "Hawk scan kernel launch");
    return MESA_OK;
}

mesa_status mesa_profile_enable(int on) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    g_prof_on = on != 0;
    return MESA_OK;
}

mesa_status mesa_profile_reset(void) {
    std::lock_guard<std::mutex> g(g_prof_mu);
    for (auto& r : g_prof_pending) {
        (void)hipEventSynchronize(r.b);
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    g_prof_pending.clear();
    for (int i = 0; i < MESA_KERNEL_COUNT; ++i) { g_prof_ms[i] = 0; g_prof_n[i] = 0; }
    return MESA_OK;
}

mesa_status mesa_profile_read(int kernel_id, double* total_ms, int64_t* launches) {
    g_err.clear();
    if (kernel_id < 0 || kernel_id >= MESA_KERNEL_COUNT || !total_ms || !launches)
        return fail(MESA_ERR_INVALID_ARGUMENT, "bad kernel id %d or null output", kernel_id);
    std::lock_guard<std::mutex> g(g_prof_mu);
    mesa_status st = MESA_OK;
    for (auto& r : g_prof_pending) {
        float ms = 0.f;
        hipError_t e = hipEventSynchronize(r.b);
        if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.a, r.b);
        if (e != hipSuccess && st == MESA_OK) st = hip_fail(e, "profiling event");
        g_prof_ms[r.kid] += ms;
        g_prof_n[r.kid] += 1;
        (void)hipEventDestroy(r.a);
        (void)hipEventDestroy(r.b);
    }
    g_prof_pending.clear();
    *total_ms = g_prof_ms[kernel_id];
    *launches = g_prof_n[kernel_id];
    return st;
}

const char* mesa_kernel_name(int kernel_id) {
    switch (kernel_id) {
        case MESA_KERNEL_CHUNK_STATES: return "chunk_states_kernel";
        case MESA_KERNEL_CG_OUTPUT: return "cg_output_kernel";
        case MESA_KERNEL_DECODE: return "decode_kernel";
        case MESA_KERNEL_QK_PREPROCESS: return "qk_preprocess_kernel";
        case MESA_KERNEL_BWD_ADJOINT: return "bwd_adjoint_kernel";
        case MESA_KERNEL_BWD_STATES: return "bwd_states_kernel";
        case MESA_KERNEL_BWD_KV: return "bwd_kv_kernel";
        case MESA_KERNEL_BWD_GATE: return "bwd_gate_kernel";
        case MESA_KERNEL_HAWK: return "hawk_kernels";
    }
    return "unknown";
}

}  // extern "C"
