// Host-side plumbing shared by the translation units of libquasar: launch
// plans (pure functions of the problem shape) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace quasar {

constexpr int kNumCU = 256;          // MI355X: 256 compute units in 8 XCDs
constexpr size_t kWsAlign = 256;     // alignment of every workspace sub-buffer

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// ---------------------------------------------------------------------------
// W8A8 linear plan.
//
// The output is cut into 16-channel tiles (one MFMA row block).  K is cut into
// 64-wide chunks (one MFMA K step).  A workgroup owns one (tile, K-split) pair;
// its `waves` wavefronts each own up to `chunks_per_wave` consecutive chunks of
// that split, stream the matching INT8 weight rows straight into MFMA operand
// registers, and reduce their partial sums in LDS.  When a tile is split
// across `splits` workgroups, each writes its exact INT32 partial to the
// workspace and the last one to arrive (per-tile counter) sums and dequantizes.
// ---------------------------------------------------------------------------
struct LinearPlan {
  int64_t M, N, K;
  int mb;               // 16-token column blocks: ceil(M / 16)
  int tiles;            // ceil(N / 16)
  int nch;              // ceil(K / 64)
  int chunks_per_wave;  // compile-time unroll of the weight stream (kernel template)
  int splits;           // workgroups per tile along K
  int chunks_per_split;
  int waves;            // wavefronts per workgroup
  // workspace layout (byte offsets)
  size_t off_qx, off_sx, off_counters, off_partials, bytes;
};

LinearPlan plan_linear(int64_t M, int64_t N, int64_t K);

// ---------------------------------------------------------------------------
// Accept plan: each logits row is cut into `chunks` pieces of `chunk_len`.
// ---------------------------------------------------------------------------
struct AcceptPlan {
  int64_t B, k, V, rows;
  int chunk_len, chunks;
  size_t off_max, off_idx, off_sum, bytes;
};

AcceptPlan plan_accept(int64_t B, int64_t k, int64_t V);

// ---------------------------------------------------------------------------
// Launchers (return the hipError_t of the launch).
// ---------------------------------------------------------------------------
hipError_t launch_quantize_weights(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                   int8_t* wq, float* w_scale, hipStream_t st);

// Smooth + quantize activations; also zeroes `zero_words` int32 words at
// `zero_ptr` (the split-K counters of the following GEMM), when non-null.
hipError_t launch_quantize_activations(const uint16_t* x, const float* s, int64_t M, int64_t K,
                                       int8_t* qx, float* sx, float* xs_out, int32_t* zero_ptr,
                                       int64_t zero_words, hipStream_t st);

hipError_t launch_gemm(const LinearPlan& p, const int8_t* qx, const float* sx, const int8_t* wq,
                       const float* w_scale, uint16_t* y, int32_t* acc_out, int32_t* counters,
                       int32_t* partials, hipStream_t st);

hipError_t launch_accept(const AcceptPlan& p, const uint16_t* logits, const int32_t* draft,
                         float temperature, const float* uniforms, int32_t* accept_len,
                         int32_t* next_token, int32_t* argmax_out, float* p_draft_out,
                         void* workspace, hipStream_t st);

}  // namespace quasar
