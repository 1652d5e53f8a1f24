/*
 * mesa.h -- C ABI of the MI355X (gfx950) Mesa-layer library (libmesa.so).
 *
 * The operation is the Mesa layer of the MesaNet summary page
 * (gist.science, paper 2506.05233), section "A Camada Mesa":
 *   - displayed objective: Phi_t = argmin 1/2 sum_{t'<=t} zeta_{tt'}
 *     |v_t' - Phi k_t'|^2 + 1/2 Tr(Phi Lambda Phi^T), zeta_{tt'} the cumulative
 *     forget factors, Lambda symmetric positive definite;
 *   - output Delta_t = Phi_t q_t = G_t q*_t, q*_t = (H_t + Lambda)^{-1} q_t,
 *     solved by Conjugate Gradient;
 *   - bullet "Paralelizacao": CG over all time steps is a gated-linear-attention
 *     pass, run chunk-parallel with the states H_t, G_t (O(T) forward, O(1)
 *     per decoded token);
 *   - bullet "Computacao Dinamica": the CG iteration count needed to meet a
 *     stopping criterion varies per token.
 *
 * Concretely, per batch row b, head h and token t (readings of the page):
 *   H_t = gamma_t H_{t-1} + k_t k_t^T,  G_t = gamma_t G_{t-1} + v_t k_t^T,
 *   H_0 = G_0 = 0  (i.e. zeta_{tt'} = prod_{s=t'+1..t} gamma_s);
 *   Lambda = diag(lambda[h, :]);
 *   x = CG on (H_t + Lambda) x = q_t from x0 = 0, at most max_iters updates;
 *       when tol > 0 a token stops before an update once
 *       |r|_2 / |q_t|_2 < tol (r the recursively updated residual);
 *       tol == 0 makes exactly max_iters updates; r^T r == 0 or p^T A p <= 0
 *       also stop; q_t == 0 gives x = 0 and 0 iterations;
 *   out_t = G_t x,  iters_t = number of CG updates made.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers (hipMalloc / torch CUDA memory),
 *     contiguous row-major, 16-byte aligned.  The caller owns every buffer;
 *     the library allocates nothing and keeps no state between calls, except
 *     the optional profiling records below.
 *   - Work is enqueued asynchronously on `stream` (a hipStream_t; NULL = the
 *     default stream).  Results are valid once the caller synchronises.
 *   - All arguments are validated on the host before anything is enqueued;
 *     on error nothing is enqueued.  Device data preconditions (0 < gamma <= 1,
 *     lambda > 0, finite inputs) are documented, not checked.
 *   - Outputs must not alias inputs.  Nothing aborts; no C++ exception
 *     crosses the ABI.  Errors return a mesa_status; the thread-local text
 *     from mesa_last_error_message() says which argument was wrong.
 *   - Supported sizes: d_k == d_v in {16, 32, 64, 128}; chunk in {16, 32, 64};
 *     any T >= 0 (a ragged last chunk is handled); 0 <= max_iters <= 4096.
 */
#ifndef MESA_H
#define MESA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MESA_ABI_VERSION 1

typedef enum {
    MESA_OK = 0,
    MESA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, tol < 0 or NaN, misaligned */
    MESA_ERR_UNSUPPORTED = 2,        /* valid but not built: d, chunk or d_k != d_v      */
    MESA_ERR_WORKSPACE_TOO_SMALL = 3,
    MESA_ERR_HIP = 4                 /* a HIP runtime call failed (text in the message)  */
} mesa_status;

typedef enum {
    MESA_DTYPE_F32 = 0,              /* q, k, v stored as float32                        */
    MESA_DTYPE_BF16 = 1              /* q, k, v stored as bfloat16; vectors, states and
                                        sums in fp32.  The chunk states' products are exact
                                        (bf16 MFMAs on three-part bf16 splits).  The CG and
                                        output products (d >= 32, either dtype) run as fp16
                                        MFMAs on two-part splits: each operand group is
                                        scaled by a power of two and held as hi + lo to 22
                                        bits, and a product is hi.hi + hi.lo + lo.hi, within
                                        about 3 * 2^-22 of the float product                 */
} mesa_dtype;

/* Kernel ids for the optional profiling records. */
typedef enum {
    MESA_KERNEL_CHUNK_STATES = 0,    /* chunk-boundary states S^H_c, S^G_c (+ final)     */
    MESA_KERNEL_CG_OUTPUT = 1,       /* all CG iterations of a chunk + output contraction */
    MESA_KERNEL_DECODE = 2,          /* one recurrent decode step                        */
    MESA_KERNEL_QK_PREPROCESS = 3,   /* q/k convolution + normalisation                  */
    MESA_KERNEL_BWD_ADJOINT = 4,     /* backward: adjoint CG solve, per-token totals     */
    MESA_KERNEL_BWD_STATES = 5,      /* backward: reverse chunk states                   */
    MESA_KERNEL_BWD_KV = 6,          /* backward: key and value gradients                */
    MESA_KERNEL_BWD_GATE = 7,        /* backward: gate and regulariser gradients         */
    MESA_KERNEL_HAWK = 8,            /* Hawk layer recurrence (all its kernels)          */
    MESA_KERNEL_COUNT = 9
} mesa_kernel_id;

/* Library ABI version (MESA_ABI_VERSION of the build). */
int mesa_abi_version(void);

/* Static text for a status code; never NULL. */
const char *mesa_status_string(int status);

/* Thread-local detail about the last error returned on this thread ("" if none). */
const char *mesa_last_error_message(void);

/*
 * Bytes of device workspace mesa_forward needs for these sizes: the
 * chunk-boundary states S^H_c = H_{c*chunk-1} (symmetric; its upper triangle
 * of 16x16 blocks, dk (dk + 16) / 2 floats) and S^G_c (dv * dk floats), fp32,
 * per chunk and head, plus a 256-byte tail (the CG kernel's chunk-claim
 * counter).  Returns 0 if the sizes are invalid or T == 0.
 */
size_t mesa_forward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);

/*
 * Mesa-layer forward over a whole sequence (the "Paralelizacao" bullet:
 * chunkwise-parallel CG; every CG matvec over all t is one gated-linear-
 * attention pass with query p and key = value = k).
 *
 *   q, k      [B, H, T, dk]   qkv_dtype
 *   v         [B, H, T, dv]   qkv_dtype
 *   gamma     [B, H, T]       float32, 0 < gamma <= 1 (gamma at the first
 *                             token has no effect: H_0 = 0)
 *   lambda    [H, dk]         float32, lambda > 0 (shared over the batch)
 *   chunk                     GPU chunk length; results do not depend on it
 *                             beyond rounding
 *   max_iters, tol            CG cap and residual tolerance (see top)
 *   out       [B, H, T, dv]   float32, written
 *   iters     [B, H, T]       int32 CG update counts, or NULL
 *   final_H   [B, H, dk, dk]  float32 H_T, or NULL   (prefill -> decode
 *   final_G   [B, H, dv, dk]  float32 G_T, or NULL    hand-off)
 *   workspace, workspace_bytes  at least mesa_forward_workspace_bytes(...);
 *                             may be NULL/0 when max_iters == 0
 *   stream                    hipStream_t or NULL
 */
mesa_status mesa_forward(const void *q, const void *k, const void *v, int qkv_dtype,
                         const float *gamma, const float *lambda,
                         int B, int H, int T, int dk, int dv, int chunk,
                         int max_iters, float tol,
                         float *out, int32_t *iters, float *final_H, float *final_G,
                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * mesa_forward for training: the same computation (without final states),
 * and also the CG solutions the backward pass needs:
 *   x_out     [B, H, T, dk]   float32, x_t = the k-step CG solution of
 *                             (H_t + Lambda) x = q_t (0 when max_iters == 0)
 */
mesa_status mesa_forward_train(const void *q, const void *k, const void *v, int qkv_dtype,
                               const float *gamma, const float *lambda,
                               int B, int H, int T, int dk, int dv, int chunk,
                               int max_iters, float tol, float *out, int32_t *iters, float *x_out,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of the device array that mesa_forward_noalloc keeps its chunk
 * states in (64 MiB on every GPU the library runs on). */
#define MESA_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * mesa_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc):
 * the same computation and arguments without the workspace.  The chunk
 * states live in a device array of MESA_NOALLOC_SCRATCH_BYTES built into
 * the library; sizes whose mesa_forward_workspace_bytes(...) exceeds it
 * return MESA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.  The
 * call allocates nothing and records no profiling events.  Every call on a
 * GPU shares that GPU's array (the chunk-state kernel rewrites all of it
 * that a call reads, including the claim counter), so calls that overlap on
 * one GPU -- on different streams or host threads -- race; serialise them.
 */
mesa_status mesa_forward_noalloc(const void *q, const void *k, const void *v, int qkv_dtype,
                                 const float *gamma, const float *lambda,
                                 int B, int H, int T, int dk, int dv, int chunk,
                                 int max_iters, float tol,
                                 float *out, int32_t *iters, float *final_H, float *final_G,
                                 void *stream);

/*
 * Bytes of device workspace mesa_backward needs: the forward chunk states
 * (as mesa_forward_workspace_bytes counts them, without its tail), two
 * d x d reverse states per chunk and head (d^2 floats each, with d/16
 * exponents each), two floats per token, d floats per chunk, head and 16
 * tokens of the chunk, and a 256-byte tail (the adjoint kernel's chunk-claim
 * counter).  0 if invalid.
 */
size_t mesa_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk);

/*
 * Backward pass of the layer for a loss L with dL/d(out) = grad_out.  The
 * page says the layer trains in parallel but gives no gradient (section "A
 * Camada Mesa", bullet "Paralelizacao").  Reading: o_t = G_t A_t^{-1} q_t
 * (A_t = H_t + Lambda) is differentiated implicitly at the forward's CG
 * solution x_t, with the adjoint system solved by the same k-step CG:
 *   z_t = CG(A_t, G_t^T g_t)                        dL/dq_t = z_t
 *   dL/dv_i = sum_{t>=i} zeta_ti (x_t . k_i) g_t
 *   dL/dk_i = sum_{t>=i} zeta_ti [(g_t . v_i) x_t - (x_t . k_i) z_t - (z_t . k_i) x_t]
 *   dL/dlambda = -sum_{b,t} z_t (.) x_t
 *   dL/dgamma_s = (1/gamma_s) sum_{t>=s} (beta_t - a_t),
 *     beta_t = g_t . o_t - z_t . (H_t x_t),  a_i = (v_i . dL/dv_i + k_i . dL/dk_i) / 2
 * (g_t = grad_out_t).  The adjoint solve stops like the forward's, relative
 * to |G_t^T g_t|.
 *
 *   k         [B, H, T, dk]   qkv_dtype (q itself is not needed)
 *   v         [B, H, T, dv]   qkv_dtype
 *   gamma, lambda             as mesa_forward
 *   x         [B, H, T, dk]   float32, x_out of mesa_forward_train
 *   out       [B, H, T, dv]   float32, out of the same forward
 *   grad_out  [B, H, T, dv]   float32
 *   chunk, max_iters, tol     as mesa_forward (use the forward's values)
 *   grad_q, grad_k [B, H, T, dk], grad_v [B, H, T, dv], grad_gamma [B, H, T],
 *   grad_lambda [H, dk]       float32, written (grad_lambda sums the batch)
 *   z_iters   [B, H, T]       int32 update counts of the adjoint solve, or NULL
 *   workspace, workspace_bytes  at least mesa_backward_workspace_bytes(...)
 * Sizes and errors as mesa_forward.  Outputs must not alias inputs.
 */
mesa_status mesa_backward(const void *k, const void *v, int qkv_dtype,
                          const float *gamma, const float *lambda,
                          const float *x, const float *out, const float *grad_out,
                          int B, int H, int T, int dk, int dv, int chunk, int max_iters, float tol,
                          float *grad_q, float *grad_k, float *grad_v, float *grad_gamma,
                          float *grad_lambda, int32_t *z_iters,
                          void *workspace, size_t workspace_bytes, void *stream);

/*
 * One recurrent decode step for N x H independent heads (the "Paralelizacao"
 * bullet: O(1) per-token inference on the states H_t, G_t; "Computacao
 * Dinamica": per-head dynamic stopping).  For each (n, h):
 *   H <- gamma H + k k^T;  G <- gamma G + v k^T   (in place)
 *   x  = CG on (H + diag lambda[h]) x = q  (max_iters, tol as above)
 *   out = G x
 *
 *   q, k      [N, H, dk]      qkv_dtype
 *   v         [N, H, dv]      qkv_dtype
 *   gamma     [N, H]          float32
 *   lambda    [H, dk]         float32
 *   state_H   [N, H, dk, dk]  float32, read and overwritten
 *   state_G   [N, H, dv, dk]  float32, read and overwritten
 *   out       [N, H, dv]      float32, written
 *   iters     [N, H]          int32, or NULL
 */
mesa_status mesa_decode_step(const void *q, const void *k, const void *v, int qkv_dtype,
                             const float *gamma, const float *lambda,
                             float *state_H, float *state_G,
                             int N, int H, int dk, int dv, int max_iters, float tol,
                             float *out, int32_t *iters, void *stream);

/* Start points of the warm-started decode solve. */
typedef enum {
    MESA_WARM_COLD = 0,       /* x0 = 0: the solve of mesa_decode_step                 */
    MESA_WARM_PREVIOUS = 1,   /* x0 = x_prev                                           */
    MESA_WARM_PROJECTED = 2   /* x0 = c x_prev, c = x_prev.q / x_prev.(H+Lambda) x_prev
                                 (0 when that denominator is not positive)            */
} mesa_warm_mode;

/*
 * One decode step whose CG starts from each head's previous solution: the
 * warm start that the page names as future work for the solver's cost
 * (section "Significancia e Alegacoes").  Arguments as mesa_decode_step, plus
 *   state_x   [N, H, dk]      float32, read and overwritten: on entry the
 *                             previous step's solution x of each head (zeros
 *                             at the start of a sequence), on exit this step's
 *   warm_mode                 a mesa_warm_mode
 * From x0 the CG is the same method with r0 = q - (H + Lambda) x0; the stop
 * test still compares |r| with |q|, a zero q still gives x = 0 and 0
 * iterations, and iters counts the updates made after x0.  The projected
 * start is the multiple of x_prev closest to the solution in the energy
 * norm, so it is never further from it, in that norm, than the cold start.
 * out = G x as before.  state_x must not alias any other argument.
 */
mesa_status mesa_decode_step_warm(const void *q, const void *k, const void *v, int qkv_dtype,
                                  const float *gamma, const float *lambda,
                                  float *state_H, float *state_G, float *state_x,
                                  int N, int H, int dk, int dv, int max_iters, float tol,
                                  int warm_mode, float *out, int32_t *iters, void *stream);

/*
 * Query/key pre-processing before the layer (section "Arquitetura (MesaNet)",
 * bullet "Pre-processamento": keys and queries are normalised and convolved
 * with a small window before the Mesa layer).  Reading: per head h, token t
 * and feature f, a causal convolution of width W over the tokens followed by
 * L2 normalisation of each token's vector,
 *   c_t[f] = sum_{j<W} conv_w[h][j][f] x_{t-j}[f],   y_t = c_t / |c_t|_2
 * (y_t = 0 when c_t = 0), in one pass: one read of x, one write of y.  Call
 * it once for q and once for k (each with its own weights).
 *
 *   x         [B, H, T, d]    in_dtype (mesa_dtype)
 *   conv_w    [H, W, d]       float32; j = 0 weighs the current token
 *   width     W, 1 <= W <= 8 (this build: W <= 4, else MESA_ERR_UNSUPPORTED)
 *   hist      [B, H, W-1, d]  in_dtype, the W-1 input rows before t = 0
 *                             (oldest first), or NULL for zeros
 *   hist_out  [B, H, W-1, d]  in_dtype, or NULL: receives the last W-1 rows
 *                             of hist followed by x, the hist of the next
 *                             piece (prefill, then one token per decode step)
 *   y         [B, H, T, d]    out_dtype (mesa_dtype; bfloat16 rounds to
 *                             nearest even)
 * d in {16, 32, 64, 128}; T >= 0.  y must not alias x, and hist_out must not
 * alias hist or x.  Inputs must be finite.
 */
mesa_status mesa_qk_preprocess(const void *x, int in_dtype, const float *conv_w, int width,
                               const void *hist, void *hist_out, int B, int H, int T, int d,
                               void *y, int out_dtype, void *stream);

/*
 * Recurrence of the Hawk layer that the hybrid "Hawk-Mesa" model alternates
 * with Mesa layers (section "Arquitetura (MesaNet)", bullet "Variante
 * Hibrida": LRU (Hawk) layers).  The page names the layer only; this is
 * Hawk's published real-gated linear recurrent unit, per channel d:
 *   r_t = sigmoid(ga_t),  i_t = sigmoid(gx_t),  a_t = sigmoid(lam_d)^(c r_t)
 *   h_t = a_t h_{t-1} + sqrt(1 - a_t^2) i_t x_t,   y_t = h_t
 * The gate pre-activations come from the layer's input projections, which are
 * plain matrix products outside this call.
 *
 *   x, ga, gx [B, T, D]       in_dtype (mesa_dtype)
 *   lam       [D]             float32
 *   c                         the gate's exponent scale (Hawk uses 8)
 *   h0        [B, D]          float32 state before t = 0, or NULL for zeros
 *   y         [B, T, D]       float32, written
 *   h_final   [B, D]          float32 state after the last token, or NULL
 *   workspace, workspace_bytes  at least mesa_hawk_workspace_bytes(B, T, D)
 * T >= 0; y must not alias the inputs.  Wide shapes (B * ceil(D / 64) >= 128)
 * run as one pass that reads each input once and leaves the workspace
 * untouched; narrower ones run a two-pass chunked scan that keeps per-chunk
 * summaries in the workspace.
 */
size_t mesa_hawk_workspace_bytes(int B, int T, int D);
mesa_status mesa_hawk_scan(const void *x, const void *ga, const void *gx, int in_dtype, const float *lam,
                           float c, const float *h0, int B, int T, int D, float *y, float *h_final,
                           void *workspace, size_t workspace_bytes, void *stream);

/*
 * Optional per-kernel timing (not part of the method).  While enabled, each
 * kernel launch made by the library is bracketed by two hipEvents recorded on
 * its stream.  mesa_profile_read synchronises on the recorded events, returns
 * the summed milliseconds and launch count for one kernel id since the last
 * reset, and mesa_profile_reset drops all records.  Records are process-wide
 * and guarded by a mutex.
 */
mesa_status mesa_profile_enable(int on);
mesa_status mesa_profile_read(int kernel_id, double *total_ms, int64_t *launches);
mesa_status mesa_profile_reset(void);
const char *mesa_kernel_name(int kernel_id);

#ifdef __cplusplus
}
#endif

#endif /* MESA_H */
