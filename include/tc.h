/*
 * tc.h — C ABI of libtc.so: the Tensor Cache outer-product memory and the
 * delta-rule memory on one AMD Instinct MI355X (gfx950).
 *
 * Sources: "Tensor Cache: Eviction-conditioned Associative Memory for
 * Transformers" (Methodology 1: two-level architecture; Methodology 2:
 * parallel weighted-sum scan) and "DeltaNet-family linear attention variants"
 * (DeltaNet: writing the prediction error).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Every tensor pointer is a DEVICE pointer to caller-owned, contiguous,
 *    row-major memory.  The library never allocates, frees or keeps a
 *    pointer after the call returns; kernels run asynchronously on the
 *    stream `s`, so the caller keeps every buffer alive until the stream has
 *    reached the end of the call.
 *  - q, k, v are [B, H, T, dk | dv] (or [B, H, dk | dv] for one decode step)
 *    in the input dtype `dt`; per-head lam (decay), eta (write rate) and g
 *    (gate logit) are float32 [H], shared across the batch; the L2 matrix A
 *    is float32 [B, H, dk, dv]; the delta-rule state S is float32
 *    [B, H, dv, dk].  Outputs are always float32.
 *  - Supported shapes: dk == dv in {16, 32, 64, 128}, chunk == 64, W >= 1,
 *    B, H, T >= 0 (the backward passes and the fact memories state their own).  B, H or T equal to 0 is a valid
 *    empty call.  Anything else returns TC_ERR_UNSUPPORTED or
 *    TC_ERR_INVALID_ARG.
 *  - All argument checks run before any HIP call.  Values that live in
 *    device memory (lam, eta, g, beta, pos) cannot be checked without a
 *    synchronisation: lam and beta must lie in [0, 1] and pos must be >= 0;
 *    the Python binding checks them.  Nothing throws across the ABI.
 *  - On a non-OK status, tc_last_error() returns a message for the calling
 *    thread; nothing has been launched unless the status is TC_ERR_HIP.
 *  - Calls are stream-ordered and keep no state between calls; two calls
 *    that write the same buffers must not overlap.
 */
#ifndef TC_H_
#define TC_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TC_OK = 0,
  TC_ERR_INVALID_ARG = 1, /* null pointer, negative size, W < 1, ...          */
  TC_ERR_UNSUPPORTED = 2, /* valid but not implemented: d, chunk, dtype        */
  TC_ERR_WORKSPACE = 3,   /* ws_bytes smaller than the *_workspace_bytes query */
  TC_ERR_HIP = 4,         /* a HIP launch failed; message holds the HIP error  */
  TC_ERR_INTERNAL = 5
} tc_status;

typedef enum { TC_F32 = 0, TC_BF16 = 1 } tc_dtype; /* input dtype of q, k, v (and the ring) */

/* ---------------------------------------------------------------------------
 * Prefill scan of the L2 memory (Tensor Cache, Methodology 1 write/read and
 * Methodology 2 parallel scan).
 *
 * Starting from an empty ring and A = 0, at every step t >= W the token t-W
 * leaves the W-token window and is written, A <- lam[h] A + eta[h] k_{t-W} v_{t-W}^T;
 * then the query reads m_t = q_t A.  Equivalently
 *     m_t = sum_{i <= t-W} eta lam^((t-W)-i) <q_t, k_i> v_i,
 * evaluated in chunks of `chunk` positions, equal to the sequential writes up
 * to rounding.
 *   m        out [B, H, T, dv] float32; rows t < W are written as 0.
 *   A_final  out [B, H, dk, dv] float32 (A after the last write) or NULL.
 *            The final ring is k, v[max(0, T-W) : T] (slot t mod W), which
 *            the caller slices itself.
 *   ws       device workspace of at least tc_scan_workspace_bytes(...) bytes
 *            (may be NULL when that is 0).
 * ------------------------------------------------------------------------- */
size_t tc_scan_workspace_bytes(int B, int H, int T, int dk, int dv, int W, int chunk, tc_dtype dt);
tc_status tc_scan_forward(const void* q, const void* k, const void* v, tc_dtype dt,
                          const float* lam, const float* eta,
                          int B, int H, int T, int dk, int dv, int W, int chunk,
                          float* m, float* A_final, void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------------------
 * tc_scan_forward without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments, results and errors as
 * tc_scan_forward, minus ws / ws_bytes.
 *
 * The scratch it needs (tc_scan_workspace_bytes(...) bytes for the same
 * arguments) comes from a 32 MiB array that the library holds on every GPU
 * it runs on, from the first call there until the process ends.  A call
 * that needs more returns TC_ERR_WORKSPACE (and launches nothing); use
 * tc_scan_forward with a workspace for those shapes.  It never calls
 * hipMalloc or hipFree.
 *
 * Every call on one GPU shares that GPU's array, and each call overwrites
 * the part it uses: calls that can overlap on one GPU (different streams,
 * different host threads without ordering) race and must not be issued.
 * The stream must belong to the current device.
 * ------------------------------------------------------------------------- */
tc_status tc_scan_forward_noalloc(const void* q, const void* k, const void* v, tc_dtype dt,
                                  const float* lam, const float* eta,
                                  int B, int H, int T, int dk, int dv, int W, int chunk,
                                  float* m, float* A_final, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Backward of the L2 read (Tensor Cache, Methodology 1 and 2: lam and eta
 * are learned per head), optionally through the gate of the fused layer
 * (Methodology 1, fusion: y = y_local + sigmoid(g) m with g learned per head).
 *   g == NULL: dm is the cotangent of m as returned by tc_scan_forward for the
 *     same arguments; the gradients are those of L = sum_t <dm_t, m_t>.
 *   g != NULL ([H] float32 gate logits): dm is the cotangent dy of the gated
 *     branch sigmoid(g) m; the gradients are those of L = sum_t <dy_t,
 *     sigmoid(g) m_t>, and dg [H] receives dL/dg.  y_local's own gradients
 *     are not computed here.  g and dg are given together or not at all.
 * A_final takes no gradient.
 *   dm       [B, H, T, dv] float32 (rows t < W are ignored: m is 0 there).
 *   dq, dk   out [B, H, T, dk] float32; dv out [B, H, T, dv] float32
 *            (dq rows t < W and dk, dv rows t >= T - W are 0).
 *   dlam, deta (and dg) out [H] float32, summed over the batch.
 *   ws       at least tc_scan_backward_workspace_bytes(...) bytes (may be NULL
 *            when that is 0).
 * Supported: dk == dv in {16, 32, 64, 128}, chunk = 64; anything else is
 * TC_ERR_UNSUPPORTED.  d = 128 runs as four d = 64 problems, one per pair of
 * column halves (q and k columns of one half, v and dm columns of one half:
 * the read is a sum of those four), whose gradients are added.  bf16 inputs:
 * dq, dlam, deta and dg come from the fp32 kernels on fp32 copies of q, k, v
 * made inside the workspace (exact), so at fp32 accuracy; with d in {64,
 * 128}, dk and dv come from two bf16 forward reads of the time-reversed
 * sequences (q, k, v and sigmoid(g) dm reversed into the workspace as bf16),
 * so at the accuracy of bf16 inputs.  The workspace query includes all of
 * these copies.  dlam at lam = 0 is the one-sided derivative.
 * ------------------------------------------------------------------------- */
size_t tc_scan_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int W, int chunk,
                                        tc_dtype dt);
tc_status tc_scan_backward(const void* q, const void* k, const void* v, tc_dtype dt,
                           const float* lam, const float* eta, const float* g,
                           int B, int H, int T, int dk, int dv, int W, int chunk,
                           const float* dm, float* dq, float* dk_out, float* dv_out,
                           float* dlam, float* deta, float* dg, void* ws, size_t ws_bytes,
                           hipStream_t s);

/* ---------------------------------------------------------------------------
 * One streaming step of the two-level cache (Tensor Cache, Methodology 1).
 *
 * For every sequence b and head h, with p = pos[b] (tokens already seen):
 *   1. if p >= W, the ring slot p mod W is occupied: its pair (k_e, v_e)
 *      is written into A: A <- lam[h] A + eta[h] k_e v_e^T;
 *   2. the new (k, v) is stored in slot p mod W;
 *   3. m = q A (after the write).
 *   q, k [B, H, dk], v [B, H, dv] in dtype dt; ring_k, ring_v in/out
 *   [B, H, W, dk | dv] in dtype dt; A in/out float32 [B, H, dk, dv];
 *   pos [B] int64 >= 0 (the caller advances it after the call);
 *   m out float32 [B, H, dv].  No workspace.
 * ------------------------------------------------------------------------- */
tc_status tc_decode_step(const void* q, const void* k, const void* v, tc_dtype dt,
                         void* ring_k, void* ring_v, float* A,
                         const float* lam, const float* eta, const int64_t* pos,
                         int B, int H, int dk, int dv, int W, float* m, hipStream_t s);

/* ---------------------------------------------------------------------------
 * One full decode step of the layer (Tensor Cache, Methodology 1: L1 exact
 * softmax over the W-slot ring, the L2 write on eviction and read, and the
 * gated fusion).  Per sequence b and head h, with p = pos[b]:
 *   1-3. exactly the steps of tc_decode_step (eviction of slot p mod W into
 *        A, the new pair into that slot, m = q A after the write);
 *   4.   y_local = sum_j softmax_j(softmax_scale <q, k_j>) v_j over the pairs
 *        the ring holds after the write: the W most recent tokens, the
 *        current one included (min(p + 1, W) of them);
 *   5.   y = y_local + sigmoid(g[h]) m.
 * Over a sequence from an empty ring and A = 0 this gives the rows of
 * tc_fused_layer.  dk == dv.
 *   q, k, v [B, H, d] in dtype dt; ring_k, ring_v in/out [B, H, W, d] in
 *   dtype dt; A in/out float32 [B, H, d, d]; lam, eta, g [H] float32;
 *   pos [B] int64 >= 0 (the caller advances it after the call);
 *   softmax_scale > 0 (the Python binding passes 1/sqrt(d) by default);
 *   y out [B, H, d] float32.  No workspace.
 * ------------------------------------------------------------------------- */
tc_status tc_decode_layer_step(const void* q, const void* k, const void* v, tc_dtype dt,
                               void* ring_k, void* ring_v, float* A,
                               const float* lam, const float* eta, const float* g,
                               const int64_t* pos, int B, int H, int dk, int dv, int W,
                               float softmax_scale, float* y, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Fused Tensor Cache layer (Tensor Cache, Methodology 1: L1 exact softmax
 * over the ring, L2 read, gated fusion).
 *
 *   y_t = sum_{j = max(0,t-W+1)}^{t} softmax_j(softmax_scale <q_t, k_j>) v_j
 *         + sigmoid(g[h]) m_t,
 * with m_t the L2 read of tc_scan_forward.  The L1 window holds the W most
 * recent tokens including token t; a token leaves the window exactly when
 * it is written into A, so each token is counted once.
 *   y        out [B, H, T, dv] float32.
 *   A_final  out [B, H, dk, dv] float32 or NULL.
 *   ws       at least tc_fused_workspace_bytes(...) bytes.
 * bf16 inputs with d in {64, 128} run on bf16 MFMA kernels (the L2 state is
 * carried in fp32; each 256-token tile's contribution passes through bf16);
 * fp32 inputs (any supported d) and bf16 with d in {16, 32} run the prefill
 * scan of tc_scan_forward and an fp32-arithmetic window softmax.
 * ------------------------------------------------------------------------- */
size_t tc_fused_workspace_bytes(int B, int H, int T, int dk, int dv, int W, int chunk, tc_dtype dt);
tc_status tc_fused_layer(const void* q, const void* k, const void* v, tc_dtype dt,
                         const float* lam, const float* eta, const float* g,
                         int B, int H, int T, int dk, int dv, int W, int chunk,
                         float softmax_scale, float* y, float* A_final,
                         void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------------------
 * The L1 cache alone: exact softmax attention over the W most recent tokens
 * (Tensor Cache, Methodology 1, L1 cache), without the L2 memory and gate:
 *   y_t = sum_{j = max(0,t-W+1)}^{t} softmax_j(softmax_scale <q_t, k_j>) v_j.
 * This is the pure sliding window the layer's cost is compared against.
 *   y        out [B, H, T, dv] float32.  No workspace.
 * bf16 inputs with d in {64, 128} run on the bf16 MFMA kernel of the fused
 * layer; other inputs on an fp32-arithmetic kernel.
 * ------------------------------------------------------------------------- */
tc_status tc_window_attention(const void* q, const void* k, const void* v, tc_dtype dt,
                              int B, int H, int T, int dk, int dv, int W, float softmax_scale,
                              float* y, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Backward of the window softmax (Tensor Cache, Methodology 1, L1 cache; the
 * pages give no backward): gradients of L = sum_t <dy_t, y_t> for the y of
 * tc_window_attention with the same arguments,
 *   dv_j = sum_t p_tj dy_t,  ds_tj = p_tj (<dy_t, v_j> - <dy_t, y_t>),
 *   dq_t = scale sum_j ds_tj k_j,  dk_j = scale sum_t ds_tj q_t,
 * with p_tj the softmax weights over the window.  bf16 inputs with d in
 * {64, 128} run on bf16 MFMA: the forward is recomputed (y and each query's
 * log-sum-exp), dy, p and ds are rounded to bf16 as MFMA operands, sums are
 * fp32 (held to the bf16-input bar).  Other inputs run in fp32 arithmetic.
 *   dy           [B, H, T, dv] float32.
 *   dq, dk, dv   out [B, H, T, d] float32.
 *   ws           at least tc_window_attention_backward_workspace_bytes(...)
 *                bytes: per query the log-sum-exp of its scores and <dy, y>,
 *                and on the MFMA path also y (fp32) and dy (bf16).
 * ------------------------------------------------------------------------- */
size_t tc_window_attention_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int W, tc_dtype dt);
tc_status tc_window_attention_backward(const void* q, const void* k, const void* v, tc_dtype dt,
                                       int B, int H, int T, int dk, int dv, int W, float softmax_scale,
                                       const float* dy, float* dq, float* dk_out, float* dv_out,
                                       void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Backward of the whole fused layer (Tensor Cache, Methodology 1, fusion:
 * y = y_local + sigmoid(g) m, with lam, eta, g learned per head): gradients
 * of L = sum_t <dy_t, y_t> for tc_fused_layer with the same arguments.  The
 * two branches see q, k, v separately, so their gradients add: the gated
 * L2-read backward of tc_scan_backward (which also gives dlam, deta, dg) and
 * the window softmax's of tc_window_attention_backward.
 *   dy               [B, H, T, dv] float32.
 *   dq, dk, dv       out [B, H, T, d] float32.
 *   dlam, deta, dg   out [H] float32, summed over the batch.
 *   ws               at least tc_fused_layer_backward_workspace_bytes(...).
 * Supported: dk == dv in {16, 32, 64, 128} (d = 128 as tc_scan_backward
 * does it), fp32 or bf16 inputs, chunk = 64.
 * The timing hook times the L2-read backward's forward-direction kernel.
 * ------------------------------------------------------------------------- */
size_t tc_fused_layer_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int W, int chunk, tc_dtype dt);
tc_status tc_fused_layer_backward(const void* q, const void* k, const void* v, tc_dtype dt,
                                  const float* lam, const float* eta, const float* g,
                                  int B, int H, int T, int dk, int dv, int W, int chunk, float softmax_scale,
                                  const float* dy, float* dq, float* dk_out, float* dv_out,
                                  float* dlam, float* deta, float* dg, void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Delta-rule scan (DeltaNet-family linear attention variants: DeltaNet
 * writes the prediction error).
 *
 *   e_t = beta_t (v_t - S_{t-1} k_t),  S_t = S_{t-1} + e_t k_t^T,  o_t = S_t q_t,
 * with S [dv, dk] starting from S0 (or zeros), evaluated in chunks of
 * `chunk` tokens (equal to the per-token rule up to rounding).
 *   beta     [B, H, T] float32 in [0, 1].
 *   S0       in [B, H, dv, dk] float32 or NULL for zeros.
 *   o        out [B, H, T, dv] float32.
 *   S_final  out [B, H, dv, dk] float32 or NULL.
 *   ws       at least delta_scan_workspace_bytes(...) bytes.
 * ------------------------------------------------------------------------- */
size_t delta_scan_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, tc_dtype dt);
tc_status delta_scan_forward(const void* q, const void* k, const void* v, tc_dtype dt,
                             const float* beta, int B, int H, int T, int dk, int dv, int chunk,
                             const float* S0, float* o, float* S_final,
                             void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Backward of the delta-rule scan (DeltaNet-family linear attention
 * variants, DeltaNet: beta_t is the learned write strength of each token).
 * Gradients of L = sum_t <do_t, o_t> + <dS_final, S_final> for the outputs
 * of delta_scan_forward with the same q, k, v, beta, S0.
 *   do       [B, H, T, dv] float32.
 *   dS_final [B, H, dv, dk] float32 or NULL (no gradient on S_final).
 *   dq, dk   out [B, H, T, dk] float32; dv out [B, H, T, dv] float32.
 *   dbeta    out [B, H, T] float32.
 *   dS0      out [B, H, dv, dk] float32 (the gradient on S0, zeros taken as
 *            S0 when it is NULL) or NULL.
 *   ws       at least delta_scan_backward_workspace_bytes(...) bytes; it holds
 *            four state-independent products of every chunk, its entering
 *            state and its exit adjoint (B*H*ceil(T/64)*(2*64*64 + 2*64*d
 *            + 2*d*d) floats), and with bf16 inputs fp32 copies of q, k, v.
 * Supported: dk == dv in {16, 32, 64, 128}, chunk = 64; anything else is
 * TC_ERR_UNSUPPORTED.  At 128 the rows of the state (the dv index, on which
 * every gradient term is a sum of per-row products) are taken 16 at a time
 * inside each chunk's gradient workgroup.  bf16 inputs are widened to fp32
 * copies inside the workspace first (exact); the workspace query includes
 * the copies.
 * ------------------------------------------------------------------------- */
size_t delta_scan_backward_workspace_bytes(int B, int H, int T, int dk, int dv, int chunk, tc_dtype dt);
tc_status delta_scan_backward(const void* q, const void* k, const void* v, tc_dtype dt,
                              const float* beta, int B, int H, int T, int dk, int dv, int chunk,
                              const float* S0, const float* d_o, const float* dS_final,
                              float* dq, float* dk_out, float* dv_out, float* dbeta, float* dS0,
                              void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------------------
 * Outer-product fact memories and their recall, float32, d in {32, 64, 128}.
 *
 * Hebbian gated-MLP fact store ("Hebbian-memory MLP stores facts in a
 * Transformer without training", simple MLP construction): with A, G
 * [m, d] (row-major; the page draws them from a Gaussian) the features are
 * phi(x) = (A x) * (G x) and the output matrix is B = (1/F) sum_i
 * v_f(i) phi(k_i)^T.
 *   hebbian_write: K [F, d], V [n_values, d], f [F] int32 (value row of each
 *     key; an index outside [0, n_values) contributes nothing) -> Bt [m, d],
 *     the transpose of B.  m must be a multiple of 64.  ws: at least
 *     hebbian_workspace_bytes(F, m, d) bytes (partial sums of B^T).
 *   hebbian_read: Q [n, d] -> out [n, d] = B phi(q) for every row q.
 * L2 read against a given matrix ("Tensor Cache", Methodology 1, m = q A):
 *   tc_memory_read: for every group g (a (b, h)), out[g] [n, d] =
 *     Q[g] [n, d] A[g] [d, d] (A as tc_scan_forward returns A_final).
 * Recall (the page's storage definition: the largest inner product with a
 * value embedding):
 *   recall_argmax: for every group g and query row R[g][i] [d], arg[g][i] =
 *     the index j of the largest <R[g][i], V[g][j]> over the group's nc
 *     candidates V[g] [nc, d] (the smallest j on a tie); best[g][i] = that
 *     inner product (best may be NULL).  groups <= 65535.
 * All pointers are device pointers owned by the caller.
 * ------------------------------------------------------------------------- */
size_t hebbian_workspace_bytes(int F, int m, int d);
tc_status hebbian_write(const float* K, const float* V, const int32_t* f, int F, int n_values,
                        const float* A, const float* G, int m, int d, float* Bt,
                        void* ws, size_t ws_bytes, hipStream_t s);
tc_status hebbian_read(const float* Q, int n, const float* A, const float* G, const float* Bt,
                       int m, int d, float* out, hipStream_t s);
tc_status tc_memory_read(const float* Q, const float* A, int groups, int n, int d, float* out,
                         hipStream_t s);
tc_status recall_argmax(const float* R, const float* V, int groups, int nq, int nc, int d,
                        int32_t* arg, float* best, hipStream_t s);

/* Workspace queries return SIZE_MAX when the arguments are invalid or
 * unsupported (tc_last_error() says why). */

/* ---------------------------------------------------------------------------
 * Timing hook for benchmarks (no counterpart on the pages).  Arms the calling
 * thread so that its next entry-point call that launches work records
 * `before` on that call's stream just before the entry point's main kernel
 * and `after` just after it:
 *   tc_fused_layer      the window-attention + L2-read kernel,
 *   tc_window_attention its only kernel,
 *   tc_window_attention_backward  its dk/dv kernel,
 *   tc_scan_forward     the output kernel,
 *   tc_scan_backward    its forward-direction kernel (dq, deta, dlam; at d = 128
 *                       that of the last of the four d = 64 pieces),
 *   delta_scan_backward its chunk-parallel gradient kernel,
 *   hebbian_write       its write kernel (not the segment sum),
 *   tc_decode_step      its only kernel,
 *   tc_decode_layer_step its only kernel,
 *   delta_scan_forward  the kernel that walks the chunks.
 * `before` and `after` are caller-created HIP events (hipEventCreate); the
 * caller reads hipEventElapsedTime(before, after) once the stream is done.
 * The hook is consumed by that call; NULL, NULL disarms it.  Exactly one
 * NULL is TC_ERR_INVALID_ARG.
 * ------------------------------------------------------------------------- */
tc_status tc_profile_next_call(hipEvent_t before, hipEvent_t after);

const char* tc_last_error(void); /* thread-local; "" when the last call was OK */
const char* tc_version(void);

#ifdef __cplusplus
}
#endif
#endif /* TC_H_ */
