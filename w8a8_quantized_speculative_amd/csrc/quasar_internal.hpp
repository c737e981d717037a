// Host-side plumbing shared by the translation units of libquasar: launch
// plans (pure functions of the problem shape) and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct quasar_chain_link;

namespace quasar {

constexpr int kNumCU = 256;          // MI355X: 256 compute units in 8 XCDs
constexpr size_t kWsAlign = 256;     // alignment of every workspace sub-buffer

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Bytes of the tile-packed INT8 weights of an N x K linear: ceil(N/16) tiles
// of ceil(K/64) chunks of 1 KB (see packed_offset in quasar_device.hpp).
inline size_t packed_weight_bytes(int64_t N, int64_t K) {
  return (size_t)((N + 15) / 16) * (size_t)((K + 63) / 64) * 1024u;
}
// 4-bit weights (K % 128 == 0): a 1 KB block per tile and pair of 64-wide chunks
inline size_t w4_packed_weight_bytes(int64_t N, int64_t K) {
  return (size_t)((N + 15) / 16) * (size_t)(K / 128) * 1024u;
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

// Optional epilogue of the one-launch linear when it computes an LM head: per
// workgroup (a contiguous range of output channels) and token row, the
// (max, lowest argmax) of the BF16 logits it wrote and, when inv_t > 0, the
// sum of exp((l - max) * inv_t).  Written at [row * grid + workgroup].
struct AcceptPartials {
  float* pmax;
  int32_t* pidx;
  float* psum;  // NULL at T = 0
  float inv_t;
};

bool fused_supported(int64_t M, int64_t K);
// The 4-bit weight variant of the one-launch linear (M <= 8, K <= 12288,
// K % 128 == 0), on the same plan.
bool w4_supported(int64_t M, int64_t K);
const char* fused_w4_kernel_name(const FusedPlan& p);
hipError_t launch_fused_w4(const FusedPlan& p, const uint16_t* x, const float* s,
                           const int8_t* wq4, const float* w_scale, uint16_t* y, int32_t* acc_out,
                           hipStream_t st);
// Name of the kernel of a one-launch plan (static storage).
const char* fused_kernel_name(const FusedPlan& p);
FusedPlan plan_fused(int64_t M, int64_t N, int64_t K);
// swiglu: the weights are in the gated order and y receives silu(gate) * up,
// [M, N / 2] (N % 16 == 0, no partials)
hipError_t launch_fused(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                        const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st,
                        const AcceptPartials* partials = nullptr, bool swiglu = false);

// ---------------------------------------------------------------------------
// Wide-window plan (9 <= M <= 128, or K > 12288): one launch of a persistent
// grid (one workgroup per compute unit, all resident at once) that quantizes
// the token rows into the workspace, passes a one-way grid barrier, and
// streams (group of tg tiles, 256 K positions) items in equal contiguous
// ranges per workgroup, finishing groups shared by two ranges through INT32
// partial sums in the workspace.
// ---------------------------------------------------------------------------
constexpr int kWideMaxGrid = 256;

struct WidePlan {
  int64_t M, N, K;
  int mb;      // 16-token blocks: ceil(M / 16), 1..8
  int ms;      // token-block split: 1, or 2 (two workgroups share a group, half the blocks each)
  int mbl;     // token blocks per workgroup: mb / ms (the kernel's MB)
  int tg;      // 16-channel tiles per group: 1, 2, 4 or 6 (2 or 3 with the split)
  int tiles;   // ceil(N / 16)
  int nch;     // ceil(K / 64)
  int groups;  // ceil(tiles / tg)
  int P;       // items per group: ceil(nch / 4)
  int U;       // groups * P
  int grid;    // workgroups (<= kWideMaxGrid, >= M)
  int wb;      // weight bits: 8 (INT8 layout) or 4 (4-bit layout)
  int lds;     // dynamic LDS bytes
  // workspace layout (byte offsets)
  size_t off_qx, off_sx, off_partials, bytes;
};

// `grid` only enters the launch; the workspace is sized for kWideMaxGrid.
WidePlan plan_wide(int64_t M, int64_t N, int64_t K, int grid, int wbits = 8);
const char* wide_kernel_name(int mb, int tg, int wbits = 8, bool split = false);
// 4-bit weights in the wide kernel: up to 96 tokens
bool wide_w4_supported(int64_t M);
int wide_tiles_per_group(int64_t M, int64_t N, int64_t K, int grid, int wbits = 8);
int wide_token_split(int64_t M, int64_t N, int64_t K, int grid, int wbits);
// Workgroups of a wide launch on the current device (0: cannot run there).
int wide_grid_for_current_device();
// The grid a wide plan launches with on the current device (0 if none fits).
int wide_launch_grid(const WidePlan& p);
// quasar_w8a8_linear_noalloc: the wide kernel's workspace in library device
// memory (one array per device); its address on the current device, or null.
constexpr size_t kNoAllocScratchBytes = (size_t)12 << 20;
void* noalloc_scratch_for_current_device();
hipError_t launch_wide(const WidePlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                       const float* w_scale, uint16_t* y, int32_t* acc_out, void* workspace,
                       hipStream_t st);

// ---------------------------------------------------------------------------
// Chained linears (M <= 8): one persistent launch over a list of links
// (quasar_chain_link), each waiting for the link that writes its input.
// ---------------------------------------------------------------------------
constexpr int kChainMaxK = 12288;
int chain_lds_bytes(int M, int Kmax);
const char* chain_kernel_name(int M);
// `partials` (optional) receive the accept partials of the LAST link, as the
// one-launch kernel's LM-head epilogue writes them ([row * G + workgroup]).
// links_dev: a device copy of the links; workspace: its flag header first.
hipError_t launch_chain(const struct quasar_chain_link* links_dev, int n, int M, int Kmax, int G,
                        void* workspace, const AcceptPartials* partials, hipStream_t st);

// ---------------------------------------------------------------------------
// Accept plan: each logits row is cut into `chunks` pieces of `chunk_len`.
// ---------------------------------------------------------------------------
constexpr int kAcceptChunk = 2048;  // widest chunk the accept finalize scans (8 per thread)

struct AcceptPlan {
  int64_t B, k, V, rows;
  int chunk_len, chunks;
  // chunk c covers logits [unit (c cq + floor(c cr / cG)), ...) of a row:
  // 2048 c for the accept kernels' own partials, a workgroup's tile range when
  // an LM-head launch produced them
  int unit, cq, cr, cG;
  size_t off_max, off_idx, off_sum, bytes;
};

AcceptPlan plan_accept(int64_t B, int64_t k, int64_t V);

// ---------------------------------------------------------------------------
// Launchers (return the hipError_t of the launch).
// ---------------------------------------------------------------------------
// gated: the rows of a [gate; up] matrix (N = 2I) in the gated order (packed
// row 16 t + i is gate row 8 t + i for i < 8, up row 8 t + i - 8 otherwise)
hipError_t launch_quantize_weights(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                   int8_t* wq, float* w_scale, hipStream_t st, bool gated = false);

hipError_t launch_quantize_weights_w4(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                      int8_t* wq4, float* w_scale, hipStream_t st);

hipError_t launch_quantize_activations(const uint16_t* x, const float* s, int64_t M, int64_t K,
                                       int8_t* qx, float* sx, float* xs_out, hipStream_t st);

hipError_t launch_accept(const AcceptPlan& p, const uint16_t* logits, const int32_t* draft,
                         float temperature, const float* uniforms, int32_t* accept_len,
                         int32_t* next_token, int32_t* argmax_out, float* p_draft_out,
                         void* workspace, hipStream_t st);

// Pass 2 alone, over partials [rows][p.chunks] made elsewhere (the LM head).
hipError_t launch_accept_finalize(const AcceptPlan& p, const uint16_t* logits,
                                  const int32_t* draft, float temperature, const float* uniforms,
                                  int32_t* accept_len, int32_t* next_token, int32_t* argmax_out,
                                  float* p_draft_out, const float* pmax, const int32_t* pidx,
                                  const float* psum, hipStream_t st);

// Decoder steps around the linears (decoder.hip).
int attn_chunks(int64_t pos0, int64_t T);
size_t attn_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t pos0);
bool attn_supported(int64_t Hq, int64_t Hkv, int64_t D, int64_t T);
hipError_t launch_embed(const int32_t* tok, const uint16_t* table, int64_t M, int64_t V, int64_t H,
                        float* h, hipStream_t st);
hipError_t launch_rmsnorm(float* h, const uint16_t* delta, const float* gamma, int64_t M, int64_t H,
                          float eps, uint16_t* out, hipStream_t st);
hipError_t launch_qk_rope_cache(const uint16_t* qkv, const float* q_gamma, const float* k_gamma,
                                int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                                int64_t pos0, int64_t Lmax, double log2_base, float eps,
                                uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache,
                                hipStream_t st);
hipError_t launch_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t pos0, int64_t Lmax,
                            uint16_t* out, void* workspace, hipStream_t st);
// silu(gate) * up from a [M, 2I] product whose columns are in the gated order
hipError_t launch_silu_mul_gated(const uint16_t* gu, int64_t M, int64_t I, uint16_t* out,
                                 hipStream_t st);
hipError_t launch_silu_mul(const uint16_t* gu, int64_t M, int64_t I, uint16_t* out, hipStream_t st);

// Diagnostic plain copy (16-byte vectors), bytes % 16 == 0.
hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t st);
// Diagnostic read-only stream of `bytes` (% 16 == 0); sink holds 1024 words.
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st);
// Zero the flag header at the start of a workspace (a kernel, so it can be
// captured in a graph).
hipError_t launch_zero_flag_header(void* workspace, hipStream_t st);

}  // namespace quasar
