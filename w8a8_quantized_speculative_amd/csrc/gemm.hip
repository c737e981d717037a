// Multi-kernel W8A8 linear for verify windows the one-launch kernel does not
// cover (M > 8 tokens, or K > 12288): the activations are quantized by the row
// quantizer into the workspace, then this INT8 x INT8 -> INT32 GEMM applies the
// BF16 dequant epilogue, or -- when K is split across workgroups -- writes exact
// INT32 partials that a small reduce kernel sums and dequantizes.
//
//   acc[m, n] = sum_k qx[m, k] * wq[n, k]                    [Quasar, pt page §2 item 3]
//   y[m, n]   = BF16(RN32(RN32(RN32(acc) * sx[m]) * sw[n]))  [pt page §2 item 4]
//
// Weights are the MFMA A operand (lane l: row tile*16 + l%16, 16 contiguous
// K positions from 64*c + 16*(l/16)), stored tile-packed so that one chunk of a
// tile is one contiguous 1 KB, streamed once with the nt cache policy through
// buffer resources whose out-of-range reads return zero (so ragged tokens and
// K tails need no branches).  The quantized activations are
// the B operand with the same K mapping, one 16-token block per MFMA.
// Wavefronts of a workgroup split K and sum their 16x16 partial tiles in LDS.
// Workgroups never wait on each other: a split tile is finished by a second
// kernel, which sees the partials through the kernel boundary.
#include "quasar_device.hpp"
#include "quasar_internal.hpp"

namespace quasar {
namespace {

constexpr int kCH = 8;  // 64-wide K chunks per wavefront (8 x 1 KB of weights in flight)

// Wavefronts per workgroup are capped so that the LDS reduction buffer
// (waves x MB x 1 KB) stays <= 32 KB and wider token blocks keep registers.
constexpr int max_waves(int mb) { return mb == 1 ? 16 : (32 / mb < 16 ? 32 / mb : 16); }

template <int MB>
__global__ __launch_bounds__(64 * max_waves(MB)) void gemm_w8a8_kernel(
    const int8_t* __restrict__ qx, const float* __restrict__ sx, const int8_t* __restrict__ wq,
    const float* __restrict__ wscale, int M, int N, int K, int splits, int chunks_per_split,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_out, int32_t* __restrict__ partials) {
  extern __shared__ int32_t red[];  // [waves][MB][64 lanes][4]

  const int tile = blockIdx.x / splits;
  const int split = blockIdx.x - tile * splits;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int nch = (K + 63) >> 6;
  const int cs0 = split * chunks_per_split;
  const int cs1 = min(nch, cs0 + chunks_per_split);
  const int c0 = cs0 + wave * kCH;

  // ---- operand streams (out-of-range offsets read as zero).  The weights are
  // tile-packed: chunk c of this tile is one contiguous 1 KB in MFMA A order,
  // zero-padded past N and K.
  const buffer_rsrc wrs = make_rsrc(wq + (size_t)tile * nch * 1024, (uint32_t)nch * 1024u);
  const buffer_rsrc xrs = make_rsrc(qx, (uint32_t)M * (uint32_t)K);
  v4i a[kCH];
#pragma unroll
  for (int j = 0; j < kCH; ++j) {
    const int c = c0 + j;
    a[j] = load16<kNonTemporal>(wrs, c < cs1 ? c * 1024 + lane * 16 : kOutOfRange);
  }

  // ---- MFMA over the token blocks
  v4i acc[MB];
#pragma unroll
  for (int tb = 0; tb < MB; ++tb) {
    acc[tb] = (v4i){0, 0, 0, 0};
    const int t = tb * 16 + r;
#pragma unroll
    for (int j = 0; j < kCH; ++j) {
      const int c = c0 + j;
      const int k = c * 64 + g * 16;
      const bool ok = c < cs1 && k < K;
      const v4i b = load16(xrs, ok ? t * K + k : kOutOfRange);
      acc[tb] = mfma_i8_16x16x64(a[j], b, acc[tb]);
    }
  }

  // ---- reduce the wavefronts' partial tiles in LDS
  const int waves = blockDim.x / kWave;
#pragma unroll
  for (int tb = 0; tb < MB; ++tb)
    *reinterpret_cast<v4i*>(&red[((wave * MB + tb) * kWave + lane) * 4]) = acc[tb];
  __syncthreads();

  const int elems = MB * 256;  // element e = tb*256 + lane*4 + reg
  if (splits > 1) {
    int32_t* mine = partials + ((size_t)tile * splits + split) * elems;
    for (int e = threadIdx.x; e < elems; e += blockDim.x) {
      int32_t tot = 0;
      for (int w = 0; w < waves; ++w) tot += red[w * elems + e];
      mine[e] = tot;
    }
    return;
  }
  for (int e = threadIdx.x; e < elems; e += blockDim.x) {
    int32_t tot = 0;
    for (int w = 0; w < waves; ++w) tot += red[w * elems + e];
    const int tb = e >> 8, ln = (e >> 2) & 63, reg = e & 3;
    const int t = tb * 16 + (ln & 15);
    const int nn = tile * 16 + 4 * (ln >> 4) + reg;
    if (t < M && nn < N) {
      float v = (float)tot;  // round to nearest even
      v = v * sx[t];
      v = v * wscale[nn];
      y[(size_t)t * N + nn] = (uint16_t)f32_to_bf16_rne(v);
      if (acc_out) acc_out[(size_t)t * N + nn] = tot;
    }
  }
}

// Sum the K-split partials of every tile (exact integers) and dequantize.
__global__ __launch_bounds__(256) void splitk_dequant_kernel(
    const int32_t* __restrict__ partials, const float* __restrict__ sx,
    const float* __restrict__ wscale, int M, int N, int mb, int splits, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out) {
  const int elems = mb * 256;
  const int tile = blockIdx.x;
  for (int e = threadIdx.x; e < elems; e += blockDim.x) {
    const int tb = e >> 8, ln = (e >> 2) & 63, reg = e & 3;
    const int t = tb * 16 + (ln & 15);
    const int nn = tile * 16 + 4 * (ln >> 4) + reg;
    if (t >= M || nn >= N) continue;
    int32_t tot = 0;
    const int32_t* base = partials + (size_t)tile * splits * elems + e;
    for (int sp = 0; sp < splits; ++sp) tot += base[(size_t)sp * elems];
    float v = (float)tot;
    v = v * sx[t];
    v = v * wscale[nn];
    y[(size_t)t * N + nn] = (uint16_t)f32_to_bf16_rne(v);
    if (acc_out) acc_out[(size_t)t * N + nn] = tot;
  }
}

}  // namespace

LinearPlan plan_linear(int64_t M, int64_t N, int64_t K) {
  LinearPlan p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.fused = fused_supported(M, K);
  p.mb = (int)((M + 15) / 16);
  if (p.mb < 1) p.mb = 1;
  p.tiles = (int)((N + 15) / 16);
  p.nch = (int)((K + 63) / 64);
  p.chunks_per_wave = kCH;
  const int wmax = max_waves(p.mb);
  const int waves_needed = (p.nch + kCH - 1) / kCH;
  int splits = (waves_needed + wmax - 1) / wmax;
  // small outputs: split K further so the grid covers the compute units
  while ((int64_t)p.tiles * splits < kNumCU && splits < waves_needed) ++splits;
  p.chunks_per_split = (p.nch + splits - 1) / splits;
  p.splits = (p.nch + p.chunks_per_split - 1) / p.chunks_per_split;
  p.waves = (p.chunks_per_split + kCH - 1) / kCH;

  size_t off = 0;
  p.off_qx = off;
  off = align_up(off + (size_t)(M * K), kWsAlign);
  p.off_sx = off;
  off = align_up(off + (size_t)M * sizeof(float), kWsAlign);
  p.off_partials = off;
  if (p.splits > 1)
    off = align_up(off + (size_t)p.tiles * p.splits * p.mb * 256 * sizeof(int32_t), kWsAlign);
  p.bytes = (M == 0 || N == 0 || p.fused) ? 0 : off;
  return p;
}

hipError_t launch_gemm(const LinearPlan& p, const int8_t* qx, const float* sx, const int8_t* wq,
                       const float* w_scale, uint16_t* y, int32_t* acc_out, int32_t* partials,
                       hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)p.tiles * p.splits)), block(p.waves * kWave);
  const size_t lds = (size_t)p.waves * p.mb * 256 * sizeof(int32_t);
  const int M = (int)p.M, N = (int)p.N, K = (int)p.K;
#define QUASAR_GEMM_CASE(MB)                                                                    \
  case MB:                                                                                      \
    gemm_w8a8_kernel<MB><<<grid, block, lds, st>>>(qx, sx, wq, w_scale, M, N, K, p.splits,      \
                                                  p.chunks_per_split, y, acc_out, partials);    \
    break;
  switch (p.mb) {
    QUASAR_GEMM_CASE(1)
    QUASAR_GEMM_CASE(2)
    QUASAR_GEMM_CASE(3)
    QUASAR_GEMM_CASE(4)
    QUASAR_GEMM_CASE(5)
    QUASAR_GEMM_CASE(6)
    QUASAR_GEMM_CASE(7)
    QUASAR_GEMM_CASE(8)
    default:
      return hipErrorInvalidValue;
  }
#undef QUASAR_GEMM_CASE
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  splitk_dequant_kernel<<<dim3((unsigned)p.tiles), dim3(256), 0, st>>>(partials, sx, w_scale, M, N,
                                                                      p.mb, p.splits, y, acc_out);
  return hipGetLastError();
}

}  // namespace quasar
