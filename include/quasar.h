/*
 * quasar.h -- C ABI of libquasar.so, the MI355X (gfx950) hot path of Quasar's
 * quantized verification: the W8A8 SmoothQuant linear that the target model
 * runs over the 1+k draft tokens of a verify step, and the accept step that
 * turns the verifier's logits into an accepted-prefix length.
 *
 * Source of the method: "Quasar: Quantized Self-Speculative Acceleration for
 * Rapid Inference via Memory-Efficient Verification" (gist.science summaries of
 * arXiv 2603.01399; pt, nl, zh and ko pages).  Citations below name the page
 * and the numbered section of its technical summary.
 *
 * Calls: quasar_quantize_weights (offline INT8 weights), quasar_w8a8_linear
 * (the verify linear), quasar_verify_accept (greedy or rejection accept), and
 * quasar_lm_head_verify (the LM head and the accept step in one call); the
 * 4-bit weight variant quasar_quantize_weights_w4 / quasar_w4a8_linear; size
 * queries and diagnostics.
 *
 * Conventions for every call
 *   - Tensors are row-major and contiguous.  BF16 values travel as uint16_t bit
 *     patterns.  Every tensor pointer is a DEVICE pointer (hipMalloc or torch
 *     CUDA memory) unless stated otherwise; sizes are element counts.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     validate their arguments on the host, then enqueue kernels on `stream`
 *     and return without synchronising.  Nothing is allocated: the caller owns
 *     every buffer, including workspaces sized by the *_workspace_bytes
 *     queries.  The only library state is one status word per device (see
 *     quasar_device_check).  Two calls may run concurrently on different
 *     streams as long as they use different workspaces.
 *   - Workspaces.  Kernels whose workgroups hand data to each other within a
 *     launch keep their flags in the first quasar_workspace_header_bytes()
 *     bytes of the workspace.  That header must be all zero before the
 *     workspace's first use (allocate it zero-filled, or call
 *     quasar_workspace_init once); the calls maintain it afterwards and never
 *     need it reset, whatever shapes and entry points use the workspace in
 *     turn (each launch advances every flag slot, whatever its grid).  A
 *     workspace belongs to one device, and to one call at a time.  The rest of
 *     a workspace may hold anything.
 *   - Argument errors are reported before any launch, as a status code; the
 *     outputs are then untouched.  A launch failure returns QUASAR_ERR_HIP.
 *     Device faults surface at the caller's next synchronisation.
 *   - Every wait of one workgroup for another is bounded.  If one gives up (a
 *     grid that could not be resident at once, e.g. next to another process's
 *     kernels, or a workspace header that was not zeroed), the kernel still
 *     finishes, that call's outputs are undefined, and the next
 *     quasar_device_check() returns QUASAR_ERR_INCOMPLETE.
 *   - Inputs must be finite.  A non-finite input is outside the contract.
 */
#ifndef QUASAR_H
#define QUASAR_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum quasar_status {
  QUASAR_OK = 0,
  QUASAR_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or value  */
  QUASAR_ERR_UNSUPPORTED = 2, /* valid in principle, outside the library's limits */
  QUASAR_ERR_WORKSPACE = 3,   /* workspace missing or smaller than required  */
  QUASAR_ERR_HIP = 4,         /* the HIP runtime rejected a launch           */
  QUASAR_ERR_INCOMPLETE = 5   /* quasar_device_check: a bounded wait gave up */
} quasar_status;

/* Detail bits of quasar_device_check: which kind of wait gave up. */
#define QUASAR_WAIT_LDS 1u       /* between wavefronts of one workgroup            */
#define QUASAR_WAIT_ROWS 2u      /* for other workgroups' quantized token rows      */
#define QUASAR_WAIT_PARTIALS 4u  /* for other workgroups' INT32 partial sums        */
#define QUASAR_WAIT_CHAIN 8u     /* for an earlier link of a chained call           */

/* Limits of the library. */
#define QUASAR_MAX_M 128      /* verify-window rows per linear call            */
#define QUASAR_MAX_K 65536    /* keeps |acc| <= K*127^2 < 2^31                 */
#define QUASAR_MAX_DRAFT 63   /* k, drafts per sequence in quasar_verify_accept */

/* Human-readable name of a status code (static storage, never NULL). */
const char* quasar_status_string(quasar_status status);

/* ABI version of this library (bumped on any change of the exported set). */
int quasar_abi_version(void);

/*
 * quasar_device_check -- waits until the current device is idle, then reads
 * and clears its status word.  QUASAR_OK if no bounded wait gave up since the
 * last check; QUASAR_ERR_INCOMPLETE otherwise, with *detail (if not NULL) the
 * QUASAR_WAIT_* bits of the waits that did (the outputs of the calls in between
 * are undefined); QUASAR_ERR_HIP if the device reports an error.  Not meant for
 * the hot loop: it synchronises the whole device.  A kernel that gives up
 * between this call's synchronisation and its read of the word (another host
 * thread launching meanwhile) is reported by the next check.
 */
quasar_status quasar_device_check(uint32_t* detail);

/*
 * quasar_debug_force_wait_expiry -- test hook, not for production: while `on`
 * is nonzero, kernels launched by this process get wait targets that can never
 * be reached and a short spin bound, so that every cross-workgroup and
 * cross-wavefront wait gives up at once and is reported by
 * quasar_device_check, while every kernel still runs to its end.  Outputs of
 * such launches are undefined (all memory accesses stay inside the call's
 * buffers).
 */
void quasar_debug_force_wait_expiry(int on);

/* Bytes of the flag header at the start of every workspace (see the
 * conventions above): 65536 (each flag word alone in a 128-byte line). */
size_t quasar_workspace_header_bytes(void);

/*
 * quasar_workspace_init -- zero the flag header of a workspace with a small
 * kernel on `stream` (not a memset, so it may be captured in a graph).  Needed
 * once per workspace before its first use unless it was allocated zeroed.
 *   workspace  device pointer, 256-byte aligned; workspace_bytes >= the header
 * Errors: WORKSPACE, HIP.
 */
quasar_status quasar_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * quasar_packed_weight_bytes -- size of the INT8 weight buffer of an N x K
 * linear: ceil(N/16) * ceil(K/64) * 1024 bytes.  Pure host function; 0 for
 * invalid sizes.
 */
size_t quasar_packed_weight_bytes(int64_t N, int64_t K);

/*
 * quasar_quantize_weights -- offline weight preparation.
 *
 * The weights are smoothed by diag(s)^-1 and quantized to INT8 once, then stay
 * resident in GPU memory [Quasar, pt page §2 execution pipeline item 1; ko page
 * §2 pipeline "offline"; zh page §2 item 2 gives Y = (W diag(s)^-1)(diag(s) X)].
 * Quantization is symmetric and uniform [pt page §2], one scale per output
 * channel:
 *     r_k  = RN32(1 / s_k)
 *     w'   = RN32(W[n,k] * r_k)                    (binary32)
 *     A_n  = max_k |w'[n,k]|
 *     w_scale[n] = RN32(A_n / 127)
 *     code[n,k]  = clamp(rint(RN32(w' * RN32(127 / A_n))), -127, 127)
 * (rint = round half to even; a row with A_n == 0 gets codes 0 and scale 0.)
 *
 * Layout of wq (tile-packed, the order the MFMA A operand is loaded in):
 * code[n,k] is stored at byte
 *     ((t * C + c) * 64 + g * 16 + r) * 16 + b
 * with t = n / 16, r = n % 16, c = k / 64, g = (k % 64) / 16, b = k % 16 and
 * C = ceil(K / 64): each 16-row x 64-column block is one contiguous 1 KB.
 * Rows n >= N of the last block and columns k >= K of the last chunk hold 0.
 *
 *   w        [N, K] bf16 bits, row-major, 16-byte aligned (in)
 *   s        [K]    float32, all > 0, 16-byte aligned     (in)
 *   N, K     N >= 0; 16 <= K <= QUASAR_MAX_K, K % 16 == 0
 *   wq       quasar_packed_weight_bytes(N, K) bytes, 16-byte aligned (out)
 *   w_scale  [N]    float32, 4-byte aligned               (out)
 * N == 0 is a no-op.  Errors: QUASAR_ERR_INVALID_ARG for null/misaligned
 * pointers or bad sizes, QUASAR_ERR_UNSUPPORTED for K > QUASAR_MAX_K.
 */
quasar_status quasar_quantize_weights(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                      int8_t* wq, float* w_scale, void* stream);

/*
 * quasar_quantize_weights_gated -- quasar_quantize_weights for the stacked
 * gate and up projections of a gated MLP, w = [W_gate; W_up] ([2I, K]), with
 * the rows stored in the gated order that quasar_w8a8_linear_swiglu expects:
 * packed row 16t + i is gate row 8t + i for i < 8 and up row 8t + i - 8
 * otherwise; w_scale follows the packed rows.  Each row is quantized exactly
 * as by quasar_quantize_weights.  N = 2I, N % 16 == 0; other arguments and
 * errors as there.
 */
quasar_status quasar_quantize_weights_gated(const uint16_t* w, const float* s, int64_t N,
                                            int64_t K, int8_t* wq, float* w_scale, void* stream);

/*
 * quasar_quantize_activations -- the online half of one linear, on its own.
 *
 * BF16 activations are smoothed by diag(s) and quantized dynamically, one
 * scale per token [Quasar, pt page §2 execution pipeline item 2; nl page §2
 * pipeline "online"]:
 *     xs[m,k]    = RN32(X[m,k] * s_k)               (binary32, never rounded to BF16)
 *     A_m        = max_k |xs[m,k]|
 *     x_scale[m] = RN32(A_m / 127)
 *     qx[m,k]    = clamp(rint(RN32(xs * RN32(127 / A_m))), -127, 127)
 * This is exactly what quasar_w8a8_linear computes internally; it is exported
 * for inspection and testing.
 *
 *   x        [M, K] bf16 bits, 16-byte aligned (in)
 *   s        [K] float32, 16-byte aligned      (in)
 *   M, K     0 <= M; 16 <= K <= QUASAR_MAX_K, K % 16 == 0
 *   qx       [M, K] int8, 16-byte aligned      (out)
 *   x_scale  [M] float32                       (out)
 *   xs_out   [M, K] float32 or NULL, 16-byte aligned (out, optional)
 */
quasar_status quasar_quantize_activations(const uint16_t* x, const float* s, int64_t M, int64_t K,
                                          int8_t* qx, float* x_scale, float* xs_out, void* stream);

/* Workspace bytes quasar_w8a8_linear needs for this shape.  Pure host
 * function, deterministic in (M, N, K).  It is 0 for an empty call and for
 * verify windows of M <= 8 tokens with K <= 12288, which keep the quantized
 * activations in on-chip memory; other shapes need the flag header (64 KB) and
 * stage the quantized activations and the INT32 partial sums of output groups
 * shared by two workgroups in the workspace (1 KB per 16-token block and
 * 64-wide K chunk, 4*M bytes, and 16 KB per 16-token block and compute unit,
 * each part rounded up to 256). */
size_t quasar_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/* Diagnostic: the kernel(s) quasar_w8a8_linear launches for an M x N x K
 * call, as the profiler names them (static storage; "" for invalid or
 * unsupported sizes).  Pure host function. */
const char* quasar_w8a8_kernel_name(int64_t M, int64_t N, int64_t K);

/*
 * quasar_w8a8_linear -- one W8A8 SmoothQuant linear over the verify window.
 *
 * Online smoothing and dynamic per-token INT8 quantization of the BF16 input
 * (as quasar_quantize_activations), an INT8 x INT8 -> INT32 product on the
 * matrix cores against the offline INT8 weights [Quasar, pt page §2 item 3;
 * zh page §2 item 3], and dequantization back to BF16 [pt page §2 item 4;
 * ko page §2 "dequantization"]:
 *     acc[m,n] = sum_k qx[m,k] * wq[n,k]               (exact int32)
 *     y[m,n]   = BF16(RN32(RN32(RN32(acc) * x_scale[m]) * w_scale[n]))
 * No bias is added.
 *
 *   x        [M, K] bf16 bits, 16-byte aligned         (in)
 *   s        [K] float32 smoothing vector, 16-byte aligned (in)
 *   wq       tile-packed INT8 weights from quasar_quantize_weights (in)
 *   w_scale  [N] float32 from quasar_quantize_weights  (in)
 *   M, N, K  0 <= M <= QUASAR_MAX_M, N >= 0, 16 <= K <= QUASAR_MAX_K, K % 16 == 0
 *   y        [M, N] bf16 bits, 2-byte aligned          (out)
 *   acc_out  [M, N] int32 or NULL                      (out, optional: the exact
 *            accumulators, for tests)
 *   workspace, workspace_bytes: device scratch of at least
 *            quasar_w8a8_workspace_bytes(M, N, K) bytes, 256-byte aligned, its
 *            flag header zeroed before first use (see the conventions above).
 *            May be NULL when that size is 0.
 * Every shape runs as one kernel launch on `stream` (quantize, GEMM and
 * dequant fused).  Windows of M <= 8 tokens with K <= 12288 use a kernel that
 * keeps the codes in on-chip memory.  Other shapes use a kernel with at most
 * one workgroup per compute unit, all resident at once (one per group of one
 * or two 16-channel weight tiles when those groups fit the device and K <=
 * 8192, else one per compute unit): its workgroups hand the quantized token
 * rows and partial sums to each other through the workspace, with flags in its
 * header.  Such calls on different streams with different
 * workspaces may overlap; a wait that gives up because the grid could not be
 * resident is reported by quasar_device_check.  The result does not depend on
 * the previous contents of the workspace beyond its header.
 * M == 0 or N == 0 is a no-op.  Errors: INVALID_ARG, UNSUPPORTED (M or K
 * beyond the limits, or a device with fewer than M compute units),
 * WORKSPACE, HIP.
 */
quasar_status quasar_w8a8_linear(const uint16_t* x, const float* s, const int8_t* wq,
                                 const float* w_scale, int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, int32_t* acc_out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * quasar_w8a8_linear_noalloc -- for callers that cannot allocate memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): quasar_w8a8_linear with the same arguments minus the
 * workspace, and the same results bit for bit.  Shapes that need a workspace
 * use a scratch array the library holds in device memory instead, one per
 * device, QUASAR_NOALLOC_SCRATCH_BYTES (12 MiB) large, kept until the process
 * ends; the call allocates nothing.  Every call on a device shares that
 * device's array: two such calls whose kernels overlap in time (on different
 * streams) race and their results are undefined; calls ordered on one stream
 * are safe.  Errors: as quasar_w8a8_linear, and UNSUPPORTED when the shape's
 * workspace (quasar_w8a8_workspace_bytes) exceeds the scratch -- every
 * M <= 128 with K <= 16384 fits.
 */
#define QUASAR_NOALLOC_SCRATCH_BYTES (12u << 20)
quasar_status quasar_w8a8_linear_noalloc(const uint16_t* x, const float* s, const int8_t* wq,
                                         const float* w_scale, int64_t M, int64_t N, int64_t K,
                                         uint16_t* y, int32_t* acc_out, void* stream);

/* Workspace bytes quasar_verify_accept needs (pure host function). */
size_t quasar_accept_workspace_bytes(int64_t B, int64_t k, int64_t V);

/*
 * quasar_verify_accept -- turn the verifier's BF16 logits into accepted drafts.
 *
 * The logits of the 1+k verify positions are dequantized BF16 values; they
 * feed either greedy verification at T = 0 [Quasar, ko page §4 "Qwen3 (Greedy,
 * T=0)"] or rejection sampling, which keeps the verifier's distribution exactly
 * [pt page §2 item 4; zh page §2 "lossless rejection sampling"].
 *
 * Greedy (temperature == 0): g[b,i] = lowest index of the maximum of
 *   logits[b,i,:] (compared as reals); accept_len[b] = largest L <= k with
 *   draft[b,i] == g[b,i] for all i < L; next_token[b] = g[b, L].
 * Rejection (temperature > 0): p_i = softmax(logits[b,i,:] / T); draft i is
 *   accepted while uniforms[b,i] < p_i(draft[b,i]); at the first rejection L
 *   the next token is drawn from p_L with the rejected draft removed and
 *   renormalised, otherwise from p_k, by inverse CDF in index order with
 *   uniforms[b,k]: the smallest j with cumsum_j > uniforms[b,k] * total.
 *   Arithmetic is binary32 (expf of the device library).
 * A draft id outside [0, V) is a mismatch (greedy) or has p = 0 (rejection).
 *
 *   logits      [B, k+1, V] bf16 bits (in)
 *   draft       [B, k] int32 (in; may be NULL when k == 0)
 *   B, k, V     B >= 0, 0 <= k <= QUASAR_MAX_DRAFT, V >= 1
 *   temperature 0 (greedy) or finite > 0
 *   uniforms    [B, k+1] float32 in [0, 1) (in; required when temperature > 0)
 *   accept_len  [B] int32 (out)
 *   next_token  [B] int32 (out)
 *   argmax_out  [B, k+1] int32 or NULL (out, greedy only: g)
 *   p_draft_out [B, k] float32 or NULL (out, rejection only: p_i(draft i))
 *   workspace   at least quasar_accept_workspace_bytes(B, k, V) bytes,
 *               256-byte aligned, any contents
 * B == 0 is a no-op.  Errors: INVALID_ARG (including temperature < 0 or NaN),
 * UNSUPPORTED (k too large), WORKSPACE, HIP.
 */
quasar_status quasar_verify_accept(const uint16_t* logits, const int32_t* draft, int64_t B,
                                   int64_t k, int64_t V, float temperature,
                                   const float* uniforms, int32_t* accept_len,
                                   int32_t* next_token, int32_t* argmax_out,
                                   float* p_draft_out, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* Workspace bytes quasar_lm_head_verify needs (pure host function); 0 for
 * invalid or unsupported sizes. */
size_t quasar_lm_head_verify_workspace_bytes(int64_t B, int64_t k, int64_t V, int64_t K);

/*
 * quasar_lm_head_verify -- the W8A8 LM head over the 1+k verify positions of B
 * sequences, then the verification decision on its logits, in one call.
 *
 * The final logits come out of the quantized LM head dequantized to BF16
 * [Quasar, zh page §2 item 3] and go straight to the accept step [pt page §2
 * item 4].  The results are those of quasar_w8a8_linear with M = B (k+1),
 * N = V (written to `logits`), followed by quasar_verify_accept on those
 * logits, with the same arithmetic.  When M <= 8 and K <= 12288 the LM head
 * kernel itself reduces each of its workgroups' channel ranges of every
 * logits row to (max, lowest argmax) and, at T > 0, the range's sum of
 * exp((l - max) / T), so the separate pass over the logits is skipped and one
 * small kernel takes the decisions; other shapes run the linear and both
 * accept passes.  (At T > 0 the sums are accumulated in another order than
 * quasar_verify_accept's, so p_draft may differ from its value in the last
 * binary32 bits.)
 *
 *   x, s, wq, w_scale  the LM head's inputs, as for quasar_w8a8_linear with
 *                      M = B (k+1) rows of x ordered [B, k+1] and N = V
 *   B, k, V, K  B >= 0, 0 <= k <= QUASAR_MAX_DRAFT, B (k+1) <= QUASAR_MAX_M,
 *               V >= 1, 16 <= K <= QUASAR_MAX_K, K % 16 == 0
 *   draft, temperature, uniforms, accept_len, next_token, argmax_out,
 *   p_draft_out   as for quasar_verify_accept
 *   logits      [B, k+1, V] bf16 bits (out)
 *   workspace   at least quasar_lm_head_verify_workspace_bytes(B, k, V, K)
 *               bytes, 256-byte aligned, its flag header zeroed before first use
 * B == 0 is a no-op.  Errors: INVALID_ARG, UNSUPPORTED, WORKSPACE, HIP.
 */
quasar_status quasar_lm_head_verify(const uint16_t* x, const float* s, const int8_t* wq,
                                    const float* w_scale, int64_t B, int64_t k, int64_t V,
                                    int64_t K, const int32_t* draft, float temperature,
                                    const float* uniforms, uint16_t* logits, int32_t* accept_len,
                                    int32_t* next_token, int32_t* argmax_out, float* p_draft_out,
                                    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------
 * Chained linears: the linears of a verify step in one launch.
 *
 * A verify step runs the target model's linears over the 1+k verify positions
 * one after the other, each reading what an earlier one wrote [Quasar, pt page
 * §2 execution pipeline: the verifier runs the target model once over the
 * drafts; items 2-4 for each linear].  quasar_w8a8_chain runs a list of such
 * W8A8 linears ("links") over one window of M <= 8 tokens as ONE persistent
 * kernel.  Link i computes exactly what quasar_w8a8_linear (or
 * quasar_w8a8_linear_swiglu, with QUASAR_LINK_SWIGLU) computes on its
 * arguments.  A link whose input is (a column slice of) the previous link's
 * output says so with dep = i - 1: it starts reading its input only once the
 * previous link is complete in every workgroup.  Weights do not depend on any
 * input, so the kernel keeps streaming the next link's weights from HBM across
 * each such wait: the weight stream, which bounds the step [pt page §1], does
 * not stop between links.  (On MI355X at 6 tokens the wait -- a grid-wide
 * hand-off, then every workgroup loading and quantizing the input -- costs
 * more than a kernel boundary does, so per-linear launches are faster; the
 * chain is kept for callers that cannot launch per linear.)
 * The grid is one workgroup per compute unit, all resident at once (see the
 * conventions on bounded waits).
 * --------------------------------------------------------------------------- */
#define QUASAR_LINK_SWIGLU 1u  /* weights from quasar_quantize_weights_gated;
                                  y receives silu(gate) * up, [M, N/2] */
#define QUASAR_CHAIN_MAX_LINKS 4096

typedef struct quasar_chain_link {
  const uint16_t* x;      /* [M, ldx] bf16 input rows; 16-byte aligned                    */
  const float* s;         /* [K] smoothing vector; 16-byte aligned                         */
  const int8_t* wq;       /* packed INT8 weights (quasar_quantize_weights, or _gated); 16 B */
  const float* w_scale;   /* [N] weight scales; 4-byte aligned                             */
  uint16_t* y;            /* [M, N] bf16 output ([M, N/2] with SWIGLU); 8-byte aligned     */
  int32_t* acc_out;       /* [M, N] int32 accumulators or NULL (tests); NULL with SWIGLU  */
  int64_t N;              /* output channels: 16 <= N, N % 16 == 0                         */
  int64_t K;              /* 16 <= K <= 12288, K % 16 == 0                                 */
  int64_t ldx;            /* row stride of x in elements: ldx >= K, ldx % 8 == 0           */
  int32_t dep;            /* -1: x is ready before the call; i - 1: x is a column slice
                             of the previous link's y (x = y_prev + col0 with col0 % 16
                             == 0, ldx = the row length of y_prev), written in this call */
  uint32_t flags;         /* 0 or QUASAR_LINK_SWIGLU                                       */
} quasar_chain_link;

/* Workspace bytes of quasar_w8a8_chain for these links (0 if they are invalid):
 * the flag header. */
size_t quasar_w8a8_chain_workspace_bytes(const quasar_chain_link* links, int64_t n_links,
                                         int64_t M);

/*
 * quasar_w8a8_chain -- run n_links W8A8 linears over the same M-token window
 * in one launch, in order, each as quasar_w8a8_linear would (bit for bit).
 *   links      HOST array of n_links descriptors: validated here, and used to
 *              plan the launch
 *   links_dev  DEVICE copy of the same n_links descriptors (same bytes), read by
 *              the kernel; 8-byte aligned; must stay unchanged until the call
 *              has run (a graph that captures the call keeps reading it)
 *   n_links    0 <= n_links <= QUASAR_CHAIN_MAX_LINKS (0 is a no-op)
 *   M          1 <= M <= 8 (one to a few sequences' 1+k verify positions)
 *   workspace  quasar_w8a8_chain_workspace_bytes(links, n_links, M) bytes,
 *              256-byte aligned, flag header zeroed before first use
 * The links' y and acc_out must not overlap each other or any link's x, except
 * that a link with dep = i - 1 reads (a slice of) the previous link's y (the
 * library does not check overlaps).  Errors: INVALID_ARG (a link that breaks a
 * rule above; nothing is launched), UNSUPPORTED (M > 8, K > 12288, too many links, a device with too
 * few compute units, or a link feeding the next one with more than 32 tiles of
 * 16 channels per compute unit), WORKSPACE, HIP.
 */
quasar_status quasar_w8a8_chain(const quasar_chain_link* links, const quasar_chain_link* links_dev,
                                int64_t n_links, int64_t M, void* workspace,
                                size_t workspace_bytes, void* stream);

/* Workspace bytes of quasar_chain_verify for these links (0 if invalid). */
size_t quasar_chain_verify_workspace_bytes(const quasar_chain_link* links, int64_t n_links,
                                           int64_t B, int64_t k);

/*
 * quasar_chain_verify -- a whole verify step's linears and its decision: the
 * chain as quasar_w8a8_chain, whose LAST link is the LM head (M = B (k+1)
 * rows ordered [B, k+1], N = V, no SWIGLU; its y receives the logits), then
 * the accept step on those logits, as quasar_lm_head_verify does it: the LM
 * head's epilogue reduces each workgroup's channel range of every logits row
 * to (max, lowest argmax) and, at T > 0, its sum of exp((l - max) / T), and one
 * small kernel takes the decisions.  Results equal quasar_w8a8_chain followed
 * by quasar_verify_accept (at T > 0, p_draft up to the last binary32 bits).
 *   links, links_dev, n_links  as for quasar_w8a8_chain (n_links >= 1)
 *   B, k        B >= 1, 0 <= k <= QUASAR_MAX_DRAFT, B (k+1) <= 8
 *   draft, temperature, uniforms, accept_len, next_token, argmax_out,
 *   p_draft_out   as for quasar_verify_accept
 *   workspace   quasar_chain_verify_workspace_bytes(links, n_links, B, k) bytes,
 *               256-byte aligned, flag header zeroed before first use
 * Errors: as quasar_w8a8_chain and quasar_verify_accept; UNSUPPORTED when a
 * workgroup's channel range of the LM head exceeds 2048.
 */
quasar_status quasar_chain_verify(const quasar_chain_link* links,
                                  const quasar_chain_link* links_dev, int64_t n_links, int64_t B,
                                  int64_t k, const int32_t* draft, float temperature,
                                  const float* uniforms, int32_t* accept_len, int32_t* next_token,
                                  int32_t* argmax_out, float* p_draft_out, void* workspace,
                                  size_t workspace_bytes, void* stream);

/* Profiler name of the kernel quasar_w8a8_chain launches for M tokens ("" if
 * unsupported); a diagnostic for the benchmark and profiles. */
const char* quasar_w8a8_chain_kernel_name(int64_t M);

/*
 * 4-bit weight variant.  The pages name verification with fewer bits (4 or 2)
 * as future work [Quasar, pt page §5; zh page §5] without fixing a scheme; this
 * library reads it as the INT8 weight rule at 4 bits: the same smoothed
 * weights W diag(s)^-1, one symmetric scale per output channel,
 * scale = RN32(absmax / 7), codes = clamp(rint(RN32(w' * RN32(7 / absmax))),
 * -7, 7); the activations stay dynamic per-token INT8, and the product is the
 * same exact integer accumulation and dequant as quasar_w8a8_linear.  It halves
 * the resident weight bytes that bound a verify step.
 *
 * Layout of wq4 (K % 128 == 0): per 16-row tile t and pair of 64-wide chunks
 * (2c, 2c+1), a 1 KB block; byte ((t*CP + c)*64 + g*16 + r)*16 + b (CP = K/128)
 * holds the code of row 16t + r at K position 64(2c) + 16g + b in its low
 * nibble and at 64(2c+1) + 16g + b in its high nibble, as 4-bit two's
 * complement.  Rows past N hold 0.  quasar_packed_weight_bytes_w4 gives the
 * size.
 */
size_t quasar_packed_weight_bytes_w4(int64_t N, int64_t K);

/*
 * quasar_quantize_weights_w4 -- offline 4-bit weight preparation (see above).
 *   w, s, N, K, w_scale  as for quasar_quantize_weights; K % 128 == 0
 *   wq4      packed 4-bit codes, quasar_packed_weight_bytes_w4(N, K) bytes,
 *            16-byte aligned (out)
 * Errors: INVALID_ARG (including K % 128 != 0), UNSUPPORTED, HIP.
 */
quasar_status quasar_quantize_weights_w4(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                         int8_t* wq4, float* w_scale, void* stream);

/*
 * quasar_w4a8_workspace_bytes -- device workspace quasar_w4a8_linear needs for
 * M x N x K: 0 for windows of at most 8 tokens with K <= 12288 (one launch,
 * no workspace), else the wide kernel's (flag header first, zero before the
 * first use, as for quasar_w8a8_workspace_bytes).  0 also for unsupported
 * sizes (K % 128 != 0, M > 96 with 4-bit weights).
 */
size_t quasar_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * quasar_w4a8_linear -- the verify linear with 4-bit weights: y = BF16(
 * RN32(RN32(RN32(acc) * sx_m) * sw_n)) with acc = sum_k qx[m,k] * qw4[n,k]
 * exact, qx the dynamic per-token INT8 codes of RN32(x * s) as in
 * quasar_w8a8_linear.  One kernel launch.
 *   x, s, y, acc_out  as for quasar_w8a8_linear
 *   wq4, w_scale      from quasar_quantize_weights_w4
 *   M, N, K           1 <= M <= 96, N >= 0, 128 <= K <= 65536, K % 128 == 0
 *   workspace         quasar_w4a8_workspace_bytes(M, N, K) bytes, 256-byte
 *                     aligned (may be NULL when that is 0); one call at a
 *                     time per workspace
 * M == 0 or N == 0 is a no-op.  Errors: INVALID_ARG (including K % 128 != 0),
 * UNSUPPORTED (M > 96, or a window of more than 8 tokens wider than one
 * workgroup per compute unit), WORKSPACE, HIP; a bounded wait that gave up is
 * reported by quasar_device_check.
 */
quasar_status quasar_w4a8_linear(const uint16_t* x, const float* s, const int8_t* wq4,
                                 const float* w_scale, int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, int32_t* acc_out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/* Profiler name of the kernel quasar_w4a8_linear launches for M x N x K ("" if
 * unsupported); a diagnostic for the benchmark and profiles. */
const char* quasar_w4a8_kernel_name(int64_t M, int64_t N, int64_t K);

/* ---------------------------------------------------------------------------
 * Decoder steps around the W8A8 linears, for a synthetic full verify step of a
 * Qwen3-8B-shaped target model [Quasar, pt page §2 execution pipeline: the
 * verifier runs the target model once over the drafted positions; zh page §2].
 * They are not part of the quantized linear and not what the method changes;
 * they put every dependency between the linears in place, so that the
 * linears' share of a whole verify step can be measured.  Token m = b*T + i is
 * position i of the T = 1 + k verify positions of sequence b; every sequence
 * of a call sits at the same position pos0 (its cached context length).
 * Arithmetic is binary32 with one rounding per operation; tensors leaving a
 * call are BF16 except the residual stream h (float32).  Errors:
 * INVALID_ARG for null pointers, misalignment or bad sizes, UNSUPPORTED for
 * shapes outside the stated limits, HIP.
 * --------------------------------------------------------------------------- */

/*
 * quasar_embed -- h[m, :] = float(table[tokens[m], :]); a token outside [0, V)
 * gives a zero row.
 *   tokens  [M] int32 (in)      table  [V, H] bf16 (in)      h  [M, H] f32 (out)
 *   M >= 0, V >= 1, 1 <= H <= 65536
 */
quasar_status quasar_embed(const int32_t* tokens, const uint16_t* table, int64_t M, int64_t V,
                           int64_t H, float* h, void* stream);

/*
 * quasar_rmsnorm -- the residual add (when delta is not NULL) and RMSNorm:
 *     h[m, j] = RN32(h[m, j] + float(delta[m, j]))
 *     r_m     = RN32(1 / RN32(sqrt(RN32(sum_j h[m, j]^2 / H) + eps)))  (binary32 sum)
 *     out     = BF16(RN32(RN32(h[m, j] * r_m) * gamma[j]))
 *   h      [M, H] f32, 16-byte aligned (in/out)
 *   delta  [M, H] bf16, 8-byte aligned, or NULL (in)
 *   gamma  [H] f32, 16-byte aligned (in)
 *   out    [M, H] bf16, 8-byte aligned (out)
 *   M >= 0, 1 <= H <= 65536, eps > 0 and finite
 */
quasar_status quasar_rmsnorm(float* h, const uint16_t* delta, const float* gamma, int64_t M,
                             int64_t H, float eps, uint16_t* out, void* stream);

/*
 * quasar_qk_rope_cache -- after the QKV linear: per-head RMSNorm of q and k
 * (as quasar_rmsnorm over the D values of a head, weights q_gamma / k_gamma),
 * rotate-half rotary embedding of q and k at position pos0 + i (the pair
 * (j, j + D/2) turns by (pos0 + i) * rope_base^(-2j / D) radians; the angle
 * and its reduction to [0, 2 pi) are computed in binary64, its sine and
 * cosine in binary32), then k and v written into the caches at that position
 * and q into q_out.
 *   qkv      [B*T, (Hq + 2 Hkv) D] bf16: q heads, then k heads, then v heads (in)
 *   q_gamma, k_gamma  [D] f32 (in)
 *   q_out    [B*T, Hq D] bf16 (out)
 *   k_cache, v_cache  [B, Hkv, Lmax, D] bf16 (in/out: positions pos0 .. pos0+T-1
 *            written)
 *   D == 128, Hq % Hkv == 0, 0 <= pos0, pos0 + T <= Lmax, rope_base > 1
 */
quasar_status quasar_qk_rope_cache(const uint16_t* qkv, const float* q_gamma,
                                   const float* k_gamma, int64_t B, int64_t T, int64_t Hq,
                                   int64_t Hkv, int64_t D, int64_t pos0, int64_t Lmax,
                                   float rope_base, float eps, uint16_t* q_out,
                                   uint16_t* k_cache, uint16_t* v_cache, void* stream);

/* Workspace bytes of quasar_attention (0 for invalid sizes). */
size_t quasar_attention_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv,
                                        int64_t pos0);

/*
 * quasar_attention -- causal grouped-query attention of the verify positions
 * over the cache: query i of sequence b, head h, sees cached positions
 * 0 .. pos0 + i of KV head h / (Hq / Hkv);
 *     out = BF16(sum_t softmax_t(RN32(q . k_t) / sqrt(D)) v_t)
 * in binary32, the softmax split into ranges of positions merged by their
 * maxima (the result differs from one pass by rounding only).
 *   q        [B*T, Hq D] bf16 from quasar_qk_rope_cache, 16-byte aligned (in)
 *   k_cache, v_cache  as above, positions 0 .. pos0+T-1 filled, 16-byte
 *            aligned (in)
 *   out      [B*T, Hq D] bf16 (out)
 *   workspace  quasar_attention_workspace_bytes(B, T, Hq, Hkv, pos0) bytes,
 *            256-byte aligned
 *   D == 128, Hq % Hkv == 0, (Hq / Hkv) * T <= 64, pos0 + T <= Lmax
 */
quasar_status quasar_attention(const uint16_t* q, const uint16_t* k_cache,
                               const uint16_t* v_cache, int64_t B, int64_t T, int64_t Hq,
                               int64_t Hkv, int64_t D, int64_t pos0, int64_t Lmax, uint16_t* out,
                               void* workspace, size_t workspace_bytes, void* stream);

/* Workspace bytes of quasar_w8a8_linear_swiglu (0 when it needs none or for
 * invalid sizes). */
size_t quasar_w8a8_linear_swiglu_workspace_bytes(int64_t M, int64_t N, int64_t K);

/*
 * quasar_w8a8_linear_swiglu -- the gate_up W8A8 linear followed by the gated
 * MLP's activation, act = silu(gate) * up, for weights from
 * quasar_quantize_weights_gated.  The result equals quasar_w8a8_linear on the
 * same rows in [gate | up] order followed by quasar_silu_mul, bit for bit.
 * Windows of M <= 8 tokens with K <= 12288 run as one launch (the linear's
 * epilogue applies the activation: no [M, N] product is written); other shapes
 * run the wide linear into the workspace, then the activation.
 *   x, s, wq, w_scale, M, K  as for quasar_w8a8_linear
 *   N        2I, the product's width; N % 16 == 0
 *   act      [M, N / 2] bf16, 8-byte aligned (out)
 *   workspace  quasar_w8a8_linear_swiglu_workspace_bytes(M, N, K) bytes,
 *            256-byte aligned (may be NULL when that is 0)
 * Errors as quasar_w8a8_linear; INVALID_ARG for N % 16 != 0.
 */
quasar_status quasar_w8a8_linear_swiglu(const uint16_t* x, const float* s, const int8_t* wq,
                                        const float* w_scale, int64_t M, int64_t N, int64_t K,
                                        uint16_t* act, void* workspace, size_t workspace_bytes,
                                        void* stream);

/*
 * quasar_silu_mul -- the MLP activation between gate_up and down:
 *     out[m, j] = BF16(RN32(RN32(g / RN32(1 + RN32(exp(-g)))) * u)),
 *     g = gate_up[m, j], u = gate_up[m, I + j]
 *   gate_up  [M, 2I] bf16: the gate half, then the up half (in)
 *   out      [M, I] bf16 (out)
 *   M >= 0, I >= 1
 */
quasar_status quasar_silu_mul(const uint16_t* gate_up, int64_t M, int64_t I, uint16_t* out,
                              void* stream);

/*
 * quasar_stream_copy -- diagnostic, not part of the method: copies `bytes`
 * bytes from src to dst (device pointers, 16-byte aligned, bytes a multiple of
 * 16, non-overlapping) with 16-byte streaming loads and stores.  A copy of B
 * bytes moves exactly B bytes each way, which makes it the reference for
 * reading the hardware's memory byte counters.  Errors: INVALID_ARG, HIP.
 */
quasar_status quasar_stream_copy(const void* src, void* dst, size_t bytes, void* stream);

/*
 * quasar_stream_read -- diagnostic, not part of the method: reads `bytes`
 * bytes at src (16-byte aligned, a multiple of 16) with 16-byte streaming loads
 * and writes nothing meaningful (sink: 1024 words of scratch, device memory).
 * The reference rate of a read-only HBM stream, the shape of the verify
 * linears' traffic.  Errors: INVALID_ARG, HIP.
 */
quasar_status quasar_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QUASAR_H */
