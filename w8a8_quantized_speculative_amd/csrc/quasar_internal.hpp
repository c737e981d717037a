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

// Bytes of the tile-packed INT8 weights of an N x K linear: ceil(N/16) tiles
// of ceil(K/64) chunks of 1 KB (see packed_offset in quasar_device.hpp).
inline size_t packed_weight_bytes(int64_t N, int64_t K) {
  return (size_t)((N + 15) / 16) * (size_t)((K + 63) / 64) * 1024u;
}

// ---------------------------------------------------------------------------
// One-launch plan (M <= 8, K <= 12288): quantize + GEMM + dequant in one
// kernel, persistent over 16-channel tiles.  No workspace.
// ---------------------------------------------------------------------------
struct FusedPlan {
  int64_t M, N, K;
  int tiles, nch;
  int mt;     // token rows compiled for (2, 4, 6 or 8 >= M)
  int variant;  // 0: K <= 4096, 1: K <= 8192, 2: K <= 12288 (streamer/helper split)
  int waves;    // streamer + helper wavefronts per workgroup
  int grid;   // persistent workgroups
  int lds;    // dynamic LDS bytes
};

bool fused_supported(int64_t M, int64_t K);
// Name of the kernel of a one-launch plan (static storage).
const char* fused_kernel_name(const FusedPlan& p);
FusedPlan plan_fused(int64_t M, int64_t N, int64_t K);
hipError_t launch_fused(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                        const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st);

// ---------------------------------------------------------------------------
// Multi-kernel W8A8 linear plan (any M <= 128): activation quantize kernel,
// then the GEMM kernel below, then (only when K is split) a reduce kernel.
//
// The output is cut into 16-channel tiles (one MFMA row block).  K is cut into
// 64-wide chunks (one MFMA K step).  A workgroup owns one (tile, K-split) pair;
// its `waves` wavefronts each own up to `chunks_per_wave` consecutive chunks of
// that split, stream the matching INT8 weight rows straight into MFMA operand
// registers, and reduce their partial sums in LDS.  When a tile is split
// across `splits` workgroups, each writes its exact INT32 partial to the
// workspace and a reduce kernel sums the partials and dequantizes.
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
  bool fused;           // the one-launch kernel applies (then no workspace)
  // workspace layout (byte offsets)
  size_t off_qx, off_sx, off_partials, bytes;
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

hipError_t launch_quantize_activations(const uint16_t* x, const float* s, int64_t M, int64_t K,
                                       int8_t* qx, float* sx, float* xs_out, hipStream_t st);

hipError_t launch_gemm(const LinearPlan& p, const int8_t* qx, const float* sx, const int8_t* wq,
                       const float* w_scale, uint16_t* y, int32_t* acc_out, int32_t* partials,
                       hipStream_t st);

hipError_t launch_accept(const AcceptPlan& p, const uint16_t* logits, const int32_t* draft,
                         float temperature, const float* uniforms, int32_t* accept_len,
                         int32_t* next_token, int32_t* argmax_out, float* p_draft_out,
                         void* workspace, hipStream_t st);

// Diagnostic plain copy (16-byte vectors), bytes % 16 == 0.
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t st);

}  // namespace quasar
