// extern "C" entry points of libquasar.so (declared in include/quasar.h).
// Every call validates its arguments on the host first, so an argument error
// never reaches the GPU, then enqueues its kernels on the caller's stream.
#include "quasar.h"
#include "quasar_internal.hpp"
#include "quasar_sync.hpp"

#include <math.h>

using namespace quasar;

namespace {

inline bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

inline quasar_status hip_status(hipError_t e) { return e == hipSuccess ? QUASAR_OK : QUASAR_ERR_HIP; }

// Shape rules shared by the quantizers and the linear.
quasar_status check_k(int64_t K) {
  if (K <= 0 || K % 16 != 0) return QUASAR_ERR_INVALID_ARG;
  if (K > QUASAR_MAX_K) return QUASAR_ERR_UNSUPPORTED;
  return QUASAR_OK;
}

constexpr int64_t kMaxRowsPerCall = (int64_t)1 << 30;

// quasar_lm_head_verify's plan.  Fused: the one-launch linear's epilogue
// writes the accept partials (one chunk per workgroup) and only the accept
// finalize runs after it; the workspace holds the partials.  Otherwise the
// linear and both accept passes run as in the two separate calls, and the
// workspace is the linear's followed by the accept step's.
struct LmHeadPlan {
  bool fused;
  FusedPlan fp;
  AcceptPlan ap;
  size_t off_pmax, off_pidx, off_psum;  // fused
  size_t lin_bytes, off_acc;            // otherwise
  size_t bytes;
};

LmHeadPlan plan_lm_head(int64_t B, int64_t k, int64_t V, int64_t K) {
  LmHeadPlan p{};
  const int64_t M = B * (k + 1);
  p.ap = plan_accept(B, k, V);
  p.fused = fused_supported(M, K);
  if (p.fused) {
    p.fp = plan_fused(M, V, K);
    // a workgroup's channel range must fit one finalize scan
    p.fused = 16 * (p.fp.tiles / p.fp.grid + 1) <= kAcceptChunk;
  }
  if (p.fused) {
    p.ap.chunks = p.fp.grid;
    p.ap.unit = 16;
    p.ap.cq = p.fp.tiles / p.fp.grid;
    p.ap.cr = p.fp.tiles % p.fp.grid;
    p.ap.cG = p.fp.grid;
    const size_t slots = (size_t)M * p.fp.grid;
    size_t off = 0;
    p.off_pmax = off;
    off = align_up(off + slots * sizeof(float), kWsAlign);
    p.off_pidx = off;
    off = align_up(off + slots * sizeof(int32_t), kWsAlign);
    p.off_psum = off;
    off = align_up(off + slots * sizeof(float), kWsAlign);
    p.bytes = off;
  } else {
    p.lin_bytes = fused_supported(M, K) ? 0 : plan_wide(M, V, K, kWideMaxGrid).bytes;
    p.off_acc = align_up(p.lin_bytes, kWsAlign);
    p.bytes = p.off_acc + p.ap.bytes;
  }
  return p;
}

// Chained linears: validate every link on the host; the widest K sizes the
// LDS code matrix.  A link with dep = i - 1 must read a column slice of link
// i - 1's output.
quasar_status check_chain(const quasar_chain_link* links, int64_t n, int64_t M, int* kmax) {
  if (M < 1 || n < 0) return QUASAR_ERR_INVALID_ARG;
  if (M > 8 || n > QUASAR_CHAIN_MAX_LINKS) return QUASAR_ERR_UNSUPPORTED;
  if (n > 0 && !links) return QUASAR_ERR_INVALID_ARG;
  int km = 16;
  for (int64_t i = 0; i < n; ++i) {
    const quasar_chain_link& L = links[i];
    if (L.N < 16 || L.N % 16 != 0 || L.K < 16 || L.K % 16 != 0) return QUASAR_ERR_INVALID_ARG;
    if (L.K > kChainMaxK || L.N > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
    if (L.ldx < L.K || L.ldx % 8 != 0) return QUASAR_ERR_INVALID_ARG;
    if ((M - 1) * L.ldx + L.K > ((int64_t)1 << 29)) return QUASAR_ERR_UNSUPPORTED;
    if (L.dep != -1 && L.dep != i - 1) return QUASAR_ERR_INVALID_ARG;
    if (L.flags & ~QUASAR_LINK_SWIGLU) return QUASAR_ERR_INVALID_ARG;
    const bool swiglu = (L.flags & QUASAR_LINK_SWIGLU) != 0;
    if (!L.x || !L.s || !L.wq || !L.w_scale || !L.y || (swiglu && L.acc_out))
      return QUASAR_ERR_INVALID_ARG;
    if (!aligned(L.x, 16) || !aligned(L.s, 16) || !aligned(L.wq, 16) || !aligned(L.w_scale, 4) ||
        !aligned(L.y, 8) || (L.acc_out && !aligned(L.acc_out, 4)))
      return QUASAR_ERR_INVALID_ARG;
    if (L.dep >= 0) {
      // x = y of the previous link + col0, same row stride, whole columns
      const quasar_chain_link& P = links[i - 1];
      const int64_t width = (P.flags & QUASAR_LINK_SWIGLU) ? P.N / 2 : P.N;
      const int64_t col0 = (int64_t)(L.x - P.y);
      if (col0 < 0 || col0 % 16 != 0 || col0 + L.K > width || L.ldx != width)
        return QUASAR_ERR_INVALID_ARG;
    }
    if (L.K > km) km = (int)L.K;
  }
  *kmax = km;
  return QUASAR_OK;
}

size_t chain_workspace_bytes(const quasar_chain_link*, int64_t) { return kFlagHeaderBytes; }

// quasar_chain_verify's workspace: the flag header, then the LM head's accept
// partials [M][kWideMaxGrid] (max, argmax, sum of exp).
struct ChainVerifyPlan {
  size_t off_pmax, off_pidx, off_psum, bytes;
};

ChainVerifyPlan plan_chain_verify(const quasar_chain_link* links, int64_t n, int64_t M) {
  ChainVerifyPlan p{};
  const size_t slots = (size_t)M * kWideMaxGrid;
  size_t off = chain_workspace_bytes(links, n);
  p.off_pmax = off;
  off = align_up(off + slots * sizeof(float), kWsAlign);
  p.off_pidx = off;
  off = align_up(off + slots * sizeof(int32_t), kWsAlign);
  p.off_psum = off;
  off = align_up(off + slots * sizeof(float), kWsAlign);
  p.bytes = off;
  return p;
}

}  // namespace

extern "C" {

const char* quasar_status_string(quasar_status status) {
  switch (status) {
    case QUASAR_OK: return "QUASAR_OK";
    case QUASAR_ERR_INVALID_ARG: return "QUASAR_ERR_INVALID_ARG: null or misaligned pointer, or bad size/value";
    case QUASAR_ERR_UNSUPPORTED: return "QUASAR_ERR_UNSUPPORTED: size outside the library's limits";
    case QUASAR_ERR_WORKSPACE: return "QUASAR_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case QUASAR_ERR_HIP: return "QUASAR_ERR_HIP: the HIP runtime rejected a launch";
    case QUASAR_ERR_INCOMPLETE:
      return "QUASAR_ERR_INCOMPLETE: a bounded wait between workgroups gave up; outputs since the "
             "last check are undefined";
  }
  return "QUASAR_ERR_UNKNOWN";
}

int quasar_abi_version(void) { return 11; }

quasar_status quasar_device_check(uint32_t* detail) {
  uint32_t bits = 0;
  if (read_and_clear_status(&bits) != hipSuccess) return QUASAR_ERR_HIP;
  if (detail) *detail = bits;
  return bits ? QUASAR_ERR_INCOMPLETE : QUASAR_OK;
}

void quasar_debug_force_wait_expiry(int on) { set_forced_wait_expiry(on != 0); }

size_t quasar_workspace_header_bytes(void) { return kFlagHeaderBytes; }

quasar_status quasar_workspace_init(void* workspace, size_t workspace_bytes, void* stream) {
  if (!workspace || workspace_bytes < kFlagHeaderBytes || !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  return hip_status(launch_zero_flag_header(workspace, (hipStream_t)stream));
}

quasar_status quasar_quantize_weights(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                      int8_t* wq, float* w_scale, void* stream) {
  if (N < 0) return QUASAR_ERR_INVALID_ARG;
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (N > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (N == 0) return QUASAR_OK;
  if (!w || !s || !wq || !w_scale) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(s, 16) || !aligned(wq, 16) || !aligned(w_scale, 4))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_quantize_weights(w, s, N, K, wq, w_scale, (hipStream_t)stream));
}

quasar_status quasar_quantize_weights_gated(const uint16_t* w, const float* s, int64_t N,
                                            int64_t K, int8_t* wq, float* w_scale, void* stream) {
  if (N < 0 || N % 16 != 0) return QUASAR_ERR_INVALID_ARG;
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (N > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (N == 0) return QUASAR_OK;
  if (!w || !s || !wq || !w_scale) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(s, 16) || !aligned(wq, 16) || !aligned(w_scale, 4))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(
      launch_quantize_weights(w, s, N, K, wq, w_scale, (hipStream_t)stream, /*gated=*/true));
}

quasar_status quasar_quantize_activations(const uint16_t* x, const float* s, int64_t M, int64_t K,
                                          int8_t* qx, float* x_scale, float* xs_out, void* stream) {
  if (M < 0) return QUASAR_ERR_INVALID_ARG;
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (M > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (M == 0) return QUASAR_OK;
  if (!x || !s || !qx || !x_scale) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(s, 16) || !aligned(qx, 16) || !aligned(x_scale, 4) ||
      (xs_out && !aligned(xs_out, 16)))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_quantize_activations(x, s, M, K, qx, x_scale, xs_out,
                                                (hipStream_t)stream));
}

size_t quasar_packed_weight_bytes(int64_t N, int64_t K) {
  if (N <= 0 || check_k(K) != QUASAR_OK || N > kMaxRowsPerCall) return 0;
  return packed_weight_bytes(N, K);
}

size_t quasar_w8a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || check_k(K) != QUASAR_OK || M > QUASAR_MAX_M || N > kMaxRowsPerCall)
    return 0;
  if (fused_supported(M, K)) return 0;
  return plan_wide(M, N, K, kWideMaxGrid).bytes;
}

const char* quasar_w8a8_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || check_k(K) != QUASAR_OK || M > QUASAR_MAX_M || N > kMaxRowsPerCall)
    return "";
  if (fused_supported(M, K)) return fused_kernel_name(plan_fused(M, N, K));
  const WidePlan p = plan_wide(M, N, K, kWideMaxGrid);
  return wide_kernel_name(p.mbl, p.tg, 8, p.ms == 2);
}

quasar_status quasar_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream) {
  if (bytes == 0) return QUASAR_OK;
  if (!src || !sink || bytes % 16 != 0 || !aligned(src, 16) || !aligned(sink, 4))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_stream_read(src, bytes, sink, (hipStream_t)stream));
}

quasar_status quasar_stream_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (bytes == 0) return QUASAR_OK;
  if (!src || !dst || bytes % 16 != 0 || !aligned(src, 16) || !aligned(dst, 16))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_stream_copy(src, dst, bytes, (hipStream_t)stream));
}

quasar_status quasar_w8a8_linear(const uint16_t* x, const float* s, const int8_t* wq,
                                 const float* w_scale, int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, int32_t* acc_out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0) return QUASAR_ERR_INVALID_ARG;
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (M > QUASAR_MAX_M || N > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return QUASAR_OK;
  if (!x || !s || !wq || !w_scale || !y) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(s, 16) || !aligned(wq, 16) || !aligned(w_scale, 4) ||
      !aligned(y, 2) || (acc_out && !aligned(acc_out, 4)))
    return QUASAR_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (fused_supported(M, K))  // one launch, no workspace
    return hip_status(launch_fused(plan_fused(M, N, K), x, s, wq, w_scale, y, acc_out, hs));
  WidePlan p = plan_wide(M, N, K, kWideMaxGrid);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  p.grid = wide_launch_grid(p);
  if (p.grid < M) return QUASAR_ERR_UNSUPPORTED;  // one resident workgroup per token row
  return hip_status(launch_wide(p, x, s, wq, w_scale, y, acc_out, workspace, hs));
}

quasar_status quasar_w8a8_linear_noalloc(const uint16_t* x, const float* s, const int8_t* wq,
                                         const float* w_scale, int64_t M, int64_t N, int64_t K,
                                         uint16_t* y, int32_t* acc_out, void* stream) {
  if (M < 0 || N < 0) return QUASAR_ERR_INVALID_ARG;
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (M > QUASAR_MAX_M || N > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return QUASAR_OK;
  if (!x || !s || !wq || !w_scale || !y) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(s, 16) || !aligned(wq, 16) || !aligned(w_scale, 4) ||
      !aligned(y, 2) || (acc_out && !aligned(acc_out, 4)))
    return QUASAR_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (fused_supported(M, K))  // no scratch needed
    return hip_status(launch_fused(plan_fused(M, N, K), x, s, wq, w_scale, y, acc_out, hs));
  WidePlan p = plan_wide(M, N, K, kWideMaxGrid);
  if (p.bytes > kNoAllocScratchBytes) return QUASAR_ERR_UNSUPPORTED;
  void* scratch = noalloc_scratch_for_current_device();
  if (!scratch) return QUASAR_ERR_HIP;
  p.grid = wide_launch_grid(p);
  if (p.grid < M) return QUASAR_ERR_UNSUPPORTED;
  return hip_status(launch_wide(p, x, s, wq, w_scale, y, acc_out, scratch, hs));
}

size_t quasar_w8a8_linear_swiglu_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || N % 16 != 0 || check_k(K) != QUASAR_OK || M > QUASAR_MAX_M ||
      N > kMaxRowsPerCall)
    return 0;
  if (fused_supported(M, K)) return 0;
  // the wide kernel's workspace, then the gated product [M, N] BF16
  return align_up(plan_wide(M, N, K, kWideMaxGrid).bytes, kWsAlign) +
         align_up((size_t)M * N * 2, kWsAlign);
}

quasar_status quasar_w8a8_linear_swiglu(const uint16_t* x, const float* s, const int8_t* wq,
                                        const float* w_scale, int64_t M, int64_t N, int64_t K,
                                        uint16_t* act, void* workspace, size_t workspace_bytes,
                                        void* stream) {
  if (M < 0 || N < 0 || N % 16 != 0) return QUASAR_ERR_INVALID_ARG;
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (M > QUASAR_MAX_M || N > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return QUASAR_OK;
  if (!x || !s || !wq || !w_scale || !act) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(s, 16) || !aligned(wq, 16) || !aligned(w_scale, 4) ||
      !aligned(act, 8))
    return QUASAR_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (fused_supported(M, K))  // one launch: the product's epilogue applies silu(gate) * up
    return hip_status(launch_fused(plan_fused(M, N, K), x, s, wq, w_scale, act, nullptr, hs,
                                   nullptr, /*swiglu=*/true));
  WidePlan p = plan_wide(M, N, K, kWideMaxGrid);
  const size_t lin = align_up(p.bytes, kWsAlign);
  if (!workspace || workspace_bytes < lin + align_up((size_t)M * N * 2, kWsAlign) ||
      !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  p.grid = wide_launch_grid(p);
  if (p.grid < M) return QUASAR_ERR_UNSUPPORTED;
  uint16_t* gu = reinterpret_cast<uint16_t*>(static_cast<char*>(workspace) + lin);
  hipError_t e = launch_wide(p, x, s, wq, w_scale, gu, nullptr, workspace, hs);
  if (e != hipSuccess) return hip_status(e);
  return hip_status(launch_silu_mul_gated(gu, M, N / 2, act, hs));
}

size_t quasar_accept_workspace_bytes(int64_t B, int64_t k, int64_t V) {
  if (B <= 0 || k < 0 || k > QUASAR_MAX_DRAFT || V <= 0 || V > kMaxRowsPerCall) return 0;
  return plan_accept(B, k, V).bytes;
}

quasar_status quasar_verify_accept(const uint16_t* logits, const int32_t* draft, int64_t B,
                                   int64_t k, int64_t V, float temperature,
                                   const float* uniforms, int32_t* accept_len,
                                   int32_t* next_token, int32_t* argmax_out,
                                   float* p_draft_out, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  if (B < 0 || k < 0 || V <= 0) return QUASAR_ERR_INVALID_ARG;
  if (!(temperature >= 0.0f) || isinf(temperature)) return QUASAR_ERR_INVALID_ARG;  // NaN too
  if (k > QUASAR_MAX_DRAFT || V > kMaxRowsPerCall || B > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (B == 0) return QUASAR_OK;
  if (!logits || !accept_len || !next_token) return QUASAR_ERR_INVALID_ARG;
  if (k > 0 && !draft) return QUASAR_ERR_INVALID_ARG;
  if (temperature > 0.0f && !uniforms) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(logits, 2) || (draft && !aligned(draft, 4)) || !aligned(accept_len, 4) ||
      !aligned(next_token, 4) || (uniforms && !aligned(uniforms, 4)) ||
      (argmax_out && !aligned(argmax_out, 4)) || (p_draft_out && !aligned(p_draft_out, 4)))
    return QUASAR_ERR_INVALID_ARG;
  const AcceptPlan p = plan_accept(B, k, V);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  return hip_status(launch_accept(p, logits, draft, temperature, uniforms, accept_len, next_token,
                                  argmax_out, p_draft_out, workspace, (hipStream_t)stream));
}

size_t quasar_packed_weight_bytes_w4(int64_t N, int64_t K) {
  if (N <= 0 || check_k(K) != QUASAR_OK || K % 128 != 0 || N > kMaxRowsPerCall) return 0;
  return w4_packed_weight_bytes(N, K);
}

quasar_status quasar_quantize_weights_w4(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                         int8_t* wq4, float* w_scale, void* stream) {
  if (N < 0) return QUASAR_ERR_INVALID_ARG;
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (K % 128 != 0) return QUASAR_ERR_INVALID_ARG;
  if (N > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (N == 0) return QUASAR_OK;
  if (!w || !s || !wq4 || !w_scale) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(w, 16) || !aligned(s, 16) || !aligned(wq4, 16) || !aligned(w_scale, 4))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_quantize_weights_w4(w, s, N, K, wq4, w_scale, (hipStream_t)stream));
}

// 4-bit weights: the one-launch kernel of small windows (M <= 8, K <= 12288)
// without workspace, else the wide kernel (M <= 96) with one.
static bool w4_shape_ok(int64_t M, int64_t N, int64_t K) {
  return M > 0 && N > 0 && check_k(K) == QUASAR_OK && K % 128 == 0 && N <= kMaxRowsPerCall &&
         (w4_supported(M, K) || wide_w4_supported(M));
}

size_t quasar_w4a8_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (!w4_shape_ok(M, N, K) || w4_supported(M, K)) return 0;
  return plan_wide(M, N, K, kWideMaxGrid, 4).bytes;
}

quasar_status quasar_w4a8_linear(const uint16_t* x, const float* s, const int8_t* wq4,
                                 const float* w_scale, int64_t M, int64_t N, int64_t K,
                                 uint16_t* y, int32_t* acc_out, void* workspace,
                                 size_t workspace_bytes, void* stream) {
  if (M < 0 || N < 0) return QUASAR_ERR_INVALID_ARG;
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (K % 128 != 0) return QUASAR_ERR_INVALID_ARG;
  if (N > kMaxRowsPerCall || M > QUASAR_MAX_M) return QUASAR_ERR_UNSUPPORTED;
  if (M == 0 || N == 0) return QUASAR_OK;
  if (!w4_shape_ok(M, N, K)) return QUASAR_ERR_UNSUPPORTED;
  if (!x || !s || !wq4 || !w_scale || !y) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(s, 16) || !aligned(wq4, 16) || !aligned(w_scale, 4) ||
      !aligned(y, 2) || (acc_out && !aligned(acc_out, 4)))
    return QUASAR_ERR_INVALID_ARG;
  hipStream_t hs = (hipStream_t)stream;
  if (w4_supported(M, K))  // one launch, no workspace
    return hip_status(launch_fused_w4(plan_fused(M, N, K), x, s, wq4, w_scale, y, acc_out, hs));
  WidePlan p = plan_wide(M, N, K, kWideMaxGrid, 4);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  p.grid = wide_launch_grid(p);
  if (p.grid < M) return QUASAR_ERR_UNSUPPORTED;  // one resident workgroup per token row
  return hip_status(launch_wide(p, x, s, wq4, w_scale, y, acc_out, workspace, hs));
}

const char* quasar_w4a8_kernel_name(int64_t M, int64_t N, int64_t K) {
  if (!w4_shape_ok(M, N, K)) return "";
  if (w4_supported(M, K)) return fused_w4_kernel_name(plan_fused(M, N, K));
  const WidePlan p = plan_wide(M, N, K, kWideMaxGrid, 4);
  return wide_kernel_name(p.mbl, p.tg, 4, p.ms == 2);
}

size_t quasar_lm_head_verify_workspace_bytes(int64_t B, int64_t k, int64_t V, int64_t K) {
  if (B <= 0 || k < 0 || k > QUASAR_MAX_DRAFT || V <= 0 || V > kMaxRowsPerCall ||
      check_k(K) != QUASAR_OK || B * (k + 1) > QUASAR_MAX_M)
    return 0;
  return plan_lm_head(B, k, V, K).bytes;
}

quasar_status quasar_lm_head_verify(const uint16_t* x, const float* s, const int8_t* wq,
                                    const float* w_scale, int64_t B, int64_t k, int64_t V,
                                    int64_t K, const int32_t* draft, float temperature,
                                    const float* uniforms, uint16_t* logits, int32_t* accept_len,
                                    int32_t* next_token, int32_t* argmax_out, float* p_draft_out,
                                    void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || k < 0 || V <= 0) return QUASAR_ERR_INVALID_ARG;
  if (!(temperature >= 0.0f) || isinf(temperature)) return QUASAR_ERR_INVALID_ARG;  // NaN too
  quasar_status st = check_k(K);
  if (st != QUASAR_OK) return st;
  if (k > QUASAR_MAX_DRAFT || V > kMaxRowsPerCall || B > QUASAR_MAX_M ||
      B * (k + 1) > QUASAR_MAX_M)
    return QUASAR_ERR_UNSUPPORTED;
  if (B == 0) return QUASAR_OK;
  if (!x || !s || !wq || !w_scale || !logits || !accept_len || !next_token)
    return QUASAR_ERR_INVALID_ARG;
  if (k > 0 && !draft) return QUASAR_ERR_INVALID_ARG;
  if (temperature > 0.0f && !uniforms) return QUASAR_ERR_INVALID_ARG;
  if (!aligned(x, 16) || !aligned(s, 16) || !aligned(wq, 16) || !aligned(w_scale, 4) ||
      !aligned(logits, 2) || (draft && !aligned(draft, 4)) || !aligned(accept_len, 4) ||
      !aligned(next_token, 4) || (uniforms && !aligned(uniforms, 4)) ||
      (argmax_out && !aligned(argmax_out, 4)) || (p_draft_out && !aligned(p_draft_out, 4)))
    return QUASAR_ERR_INVALID_ARG;
  const LmHeadPlan p = plan_lm_head(B, k, V, K);
  if (!workspace || workspace_bytes < p.bytes || !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  hipStream_t hs = (hipStream_t)stream;
  char* ws = static_cast<char*>(workspace);
  const int64_t M = B * (k + 1);
  if (!p.fused) {
    st = quasar_w8a8_linear(x, s, wq, w_scale, M, V, K, logits, nullptr,
                            p.lin_bytes ? ws : nullptr, p.lin_bytes, stream);
    if (st != QUASAR_OK) return st;
    return quasar_verify_accept(logits, draft, B, k, V, temperature, uniforms, accept_len,
                                next_token, argmax_out, p_draft_out, ws + p.off_acc, p.ap.bytes,
                                stream);
  }
  float* pmax = reinterpret_cast<float*>(ws + p.off_pmax);
  int32_t* pidx = reinterpret_cast<int32_t*>(ws + p.off_pidx);
  float* psum = reinterpret_cast<float*>(ws + p.off_psum);
  const bool sample = temperature > 0.0f;
  const AcceptPartials parts{pmax, pidx, sample ? psum : nullptr, sample ? 1.0f / temperature : 0.0f};
  hipError_t e = launch_fused(p.fp, x, s, wq, w_scale, logits, nullptr, hs, &parts);
  if (e != hipSuccess) return QUASAR_ERR_HIP;
  return hip_status(launch_accept_finalize(p.ap, logits, draft, temperature, uniforms, accept_len,
                                           next_token, argmax_out, p_draft_out, pmax, pidx, psum,
                                           hs));
}

size_t quasar_w8a8_chain_workspace_bytes(const quasar_chain_link* links, int64_t n_links,
                                         int64_t M) {
  int kmax = 0;
  if (check_chain(links, n_links, M, &kmax) != QUASAR_OK) return 0;
  return chain_workspace_bytes(links, n_links);
}

const char* quasar_w8a8_chain_kernel_name(int64_t M) {
  if (M < 1 || M > 8) return "";
  return chain_kernel_name((int)M);
}

quasar_status quasar_w8a8_chain(const quasar_chain_link* links, const quasar_chain_link* links_dev,
                                int64_t n_links, int64_t M, void* workspace,
                                size_t workspace_bytes, void* stream) {
  int kmax = 0;
  quasar_status st = check_chain(links, n_links, M, &kmax);
  if (st != QUASAR_OK) return st;
  if (n_links == 0) return QUASAR_OK;
  if (!links_dev || !aligned(links_dev, 8)) return QUASAR_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < chain_workspace_bytes(links, n_links) ||
      !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  const int G = wide_grid_for_current_device();
  if (G < 1) return QUASAR_ERR_UNSUPPORTED;
  return hip_status(launch_chain(links_dev, (int)n_links, (int)M, kmax, G, workspace, nullptr,
                                 (hipStream_t)stream));
}

size_t quasar_chain_verify_workspace_bytes(const quasar_chain_link* links, int64_t n_links,
                                           int64_t B, int64_t k) {
  if (B < 1 || k < 0 || k > QUASAR_MAX_DRAFT || B * (k + 1) > 8 || n_links < 1) return 0;
  int kmax = 0;
  if (check_chain(links, n_links, B * (k + 1), &kmax) != QUASAR_OK) return 0;
  return plan_chain_verify(links, n_links, B * (k + 1)).bytes;
}

quasar_status quasar_chain_verify(const quasar_chain_link* links,
                                  const quasar_chain_link* links_dev, int64_t n_links, int64_t B,
                                  int64_t k, const int32_t* draft, float temperature,
                                  const float* uniforms, int32_t* accept_len, int32_t* next_token,
                                  int32_t* argmax_out, float* p_draft_out, void* workspace,
                                  size_t workspace_bytes, void* stream) {
  if (B < 1 || k < 0 || n_links < 1) return QUASAR_ERR_INVALID_ARG;
  if (!(temperature >= 0.0f) || isinf(temperature)) return QUASAR_ERR_INVALID_ARG;  // NaN too
  if (k > QUASAR_MAX_DRAFT || B * (k + 1) > 8) return QUASAR_ERR_UNSUPPORTED;
  const int64_t M = B * (k + 1);
  int kmax = 0;
  quasar_status st = check_chain(links, n_links, M, &kmax);
  if (st != QUASAR_OK) return st;
  const quasar_chain_link& head = links[n_links - 1];
  if (head.flags & QUASAR_LINK_SWIGLU) return QUASAR_ERR_INVALID_ARG;
  if (!accept_len || !next_token) return QUASAR_ERR_INVALID_ARG;
  if (k > 0 && !draft) return QUASAR_ERR_INVALID_ARG;
  if (temperature > 0.0f && !uniforms) return QUASAR_ERR_INVALID_ARG;
  if ((draft && !aligned(draft, 4)) || !aligned(accept_len, 4) || !aligned(next_token, 4) ||
      (uniforms && !aligned(uniforms, 4)) || (argmax_out && !aligned(argmax_out, 4)) ||
      (p_draft_out && !aligned(p_draft_out, 4)))
    return QUASAR_ERR_INVALID_ARG;
  if (!links_dev || !aligned(links_dev, 8)) return QUASAR_ERR_INVALID_ARG;
  const int64_t V = head.N;
  const ChainVerifyPlan cp = plan_chain_verify(links, n_links, M);
  if (!workspace || workspace_bytes < cp.bytes || !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  const int G = wide_grid_for_current_device();
  if (G < 1) return QUASAR_ERR_UNSUPPORTED;
  AcceptPlan ap = plan_accept(B, k, V);
  const int tiles = (int)((V + 15) / 16);
  if (16 * (tiles / G + 1) > kAcceptChunk) return QUASAR_ERR_UNSUPPORTED;
  ap.chunks = G;
  ap.unit = 16;
  ap.cq = tiles / G;
  ap.cr = tiles % G;
  ap.cG = G;
  char* ws = static_cast<char*>(workspace);
  float* pmax = reinterpret_cast<float*>(ws + cp.off_pmax);
  int32_t* pidx = reinterpret_cast<int32_t*>(ws + cp.off_pidx);
  float* psum = reinterpret_cast<float*>(ws + cp.off_psum);
  const bool sample = temperature > 0.0f;
  const AcceptPartials parts{pmax, pidx, sample ? psum : nullptr, sample ? 1.0f / temperature : 0.0f};
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = launch_chain(links_dev, (int)n_links, (int)M, kmax, G, workspace, &parts, hs);
  if (e != hipSuccess) return QUASAR_ERR_HIP;
  return hip_status(launch_accept_finalize(ap, head.y, draft, temperature, uniforms, accept_len,
                                           next_token, argmax_out, p_draft_out, pmax, pidx, psum,
                                           hs));
}

// ---------------------------------------------------------------------------
// Decoder steps around the linears.
// ---------------------------------------------------------------------------
namespace {
constexpr int64_t kMaxHidden = 65536;
constexpr int64_t kMaxGridY = 65535;
}  // namespace

quasar_status quasar_embed(const int32_t* tokens, const uint16_t* table, int64_t M, int64_t V,
                           int64_t H, float* h, void* stream) {
  if (M < 0 || V <= 0 || H <= 0) return QUASAR_ERR_INVALID_ARG;
  if (H > kMaxHidden || M > kMaxRowsPerCall || V > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (M == 0) return QUASAR_OK;
  if (!tokens || !table || !h || !aligned(tokens, 4) || !aligned(table, 2) || !aligned(h, 4))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_embed(tokens, table, M, V, H, h, (hipStream_t)stream));
}

quasar_status quasar_rmsnorm(float* h, const uint16_t* delta, const float* gamma, int64_t M,
                             int64_t H, float eps, uint16_t* out, void* stream) {
  if (M < 0 || H <= 0 || !(eps > 0.0f) || isinf(eps)) return QUASAR_ERR_INVALID_ARG;
  if (H > kMaxHidden || M > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (M == 0) return QUASAR_OK;
  if (!h || !gamma || !out || !aligned(h, 16) || !aligned(gamma, 16) || !aligned(out, 8) ||
      (delta && !aligned(delta, 8)))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_rmsnorm(h, delta, gamma, M, H, eps, out, (hipStream_t)stream));
}

quasar_status quasar_qk_rope_cache(const uint16_t* qkv, const float* q_gamma,
                                   const float* k_gamma, int64_t B, int64_t T, int64_t Hq,
                                   int64_t Hkv, int64_t D, int64_t pos0, int64_t Lmax,
                                   float rope_base, float eps, uint16_t* q_out,
                                   uint16_t* k_cache, uint16_t* v_cache, void* stream) {
  if (B < 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || pos0 < 0 || Lmax <= 0 || !(eps > 0.0f) ||
      isinf(eps) || !(rope_base > 1.0f) || isinf(rope_base))
    return QUASAR_ERR_INVALID_ARG;
  if (D != 128 || Hq % Hkv != 0 || pos0 + T > Lmax) return QUASAR_ERR_UNSUPPORTED;
  if (B * T > kMaxRowsPerCall || Hq + 2 * Hkv > kMaxGridY || Lmax > kMaxRowsPerCall)
    return QUASAR_ERR_UNSUPPORTED;
  if (B == 0) return QUASAR_OK;
  if (!qkv || !q_gamma || !k_gamma || !q_out || !k_cache || !v_cache || !aligned(qkv, 2) ||
      !aligned(q_gamma, 4) || !aligned(k_gamma, 4) || !aligned(q_out, 2) || !aligned(k_cache, 2) ||
      !aligned(v_cache, 2))
    return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_qk_rope_cache(qkv, q_gamma, k_gamma, B, T, Hq, Hkv, D, pos0, Lmax,
                                         log2((double)rope_base), eps, q_out, k_cache, v_cache,
                                         (hipStream_t)stream));
}

size_t quasar_attention_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv,
                                        int64_t pos0) {
  if (B <= 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || pos0 < 0 || B * T > kMaxRowsPerCall ||
      pos0 > kMaxRowsPerCall)
    return 0;
  return attn_workspace_bytes(B, T, Hq, Hkv, pos0);
}

quasar_status quasar_attention(const uint16_t* q, const uint16_t* k_cache,
                               const uint16_t* v_cache, int64_t B, int64_t T, int64_t Hq,
                               int64_t Hkv, int64_t D, int64_t pos0, int64_t Lmax, uint16_t* out,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (B < 0 || T <= 0 || Hq <= 0 || Hkv <= 0 || pos0 < 0 || Lmax <= 0)
    return QUASAR_ERR_INVALID_ARG;
  if (!attn_supported(Hq, Hkv, D, T) || pos0 + T > Lmax || B > kMaxGridY ||
      Hq > kMaxGridY || B * T > kMaxRowsPerCall || Lmax > kMaxRowsPerCall)
    return QUASAR_ERR_UNSUPPORTED;
  if (B == 0) return QUASAR_OK;
  if (!q || !k_cache || !v_cache || !out || !aligned(q, 16) || !aligned(k_cache, 16) ||
      !aligned(v_cache, 16) || !aligned(out, 2))
    return QUASAR_ERR_INVALID_ARG;
  if (!workspace || workspace_bytes < attn_workspace_bytes(B, T, Hq, Hkv, pos0) ||
      !aligned(workspace, kWsAlign))
    return QUASAR_ERR_WORKSPACE;
  return hip_status(launch_attention(q, k_cache, v_cache, B, T, Hq, Hkv, pos0, Lmax, out,
                                     workspace, (hipStream_t)stream));
}

quasar_status quasar_silu_mul(const uint16_t* gate_up, int64_t M, int64_t I, uint16_t* out,
                              void* stream) {
  if (M < 0 || I <= 0) return QUASAR_ERR_INVALID_ARG;
  if (M > kMaxGridY || I > kMaxRowsPerCall) return QUASAR_ERR_UNSUPPORTED;
  if (M == 0) return QUASAR_OK;
  if (!gate_up || !out || !aligned(gate_up, 2) || !aligned(out, 2)) return QUASAR_ERR_INVALID_ARG;
  return hip_status(launch_silu_mul(gate_up, M, I, out, (hipStream_t)stream));
}

}  // extern "C"
