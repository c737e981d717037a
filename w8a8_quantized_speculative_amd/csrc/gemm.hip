// INT8 x INT8 -> INT32 GEMM with the BF16 dequant epilogue, for the skinny
// verify window (M = B * (1 + k) tokens, usually 6..96).
//
//   acc[m, n] = sum_k qx[m, k] * wq[n, k]                    [Quasar, pt page §2 item 3]
//   y[m, n]   = BF16(RN32(RN32(RN32(acc) * sx[m]) * sw[n]))  [pt page §2 item 4]
//
// The step is bound by streaming the INT8 weights from HBM once (every weight
// byte feeds one MFMA that serves all tokens), so the kernel is organised
// around the weight stream:
//   * weights are the MFMA A operand: lane l loads 16 contiguous bytes of row
//     (tile*16 + l%16) at K offset 64*c + 16*(l/16) with one 128-bit load, so
//     one load instruction covers 16 rows x 64 contiguous bytes and each
//     wavefront keeps `kCH` such loads in flight;
//   * the quantized activations (a few KB, L2-resident) are the B operand,
//     loaded with the same K mapping, only for lanes whose token exists;
//   * wavefronts of a workgroup split K; their 16x16 INT32 partial tiles are
//     summed in LDS; a tile split across workgroups is finished by the last
//     workgroup to arrive (exact integer sums, so the order is irrelevant).
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
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_out, int32_t* __restrict__ counters,
    int32_t* __restrict__ partials) {
  extern __shared__ int32_t red[];  // [waves][MB][64 lanes][4]
  __shared__ int s_last;

  const int tile = blockIdx.x / splits;
  const int split = blockIdx.x - tile * splits;
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int r = lane & 15, g = lane >> 4;
  const int nch = (K + 63) >> 6;
  const int cs0 = split * chunks_per_split;
  const int cs1 = min(nch, cs0 + chunks_per_split);
  const int c0 = cs0 + wave * kCH;

  // ---- weight stream: all of this wavefront's loads are issued up front
  const int n = tile * 16 + r;
  const bool row_ok = n < N;
  const int8_t* wrow = wq + (size_t)(row_ok ? n : 0) * (size_t)K;
  v4i a[kCH];
#pragma unroll
  for (int j = 0; j < kCH; ++j) {
    const int c = c0 + j;
    const int k = c * 64 + g * 16;
    a[j] = (v4i){0, 0, 0, 0};
    if (c < cs1 && row_ok && k < K) a[j] = *reinterpret_cast<const v4i*>(wrow + k);
  }

  // ---- MFMA over the token blocks
  v4i acc[MB];
#pragma unroll
  for (int tb = 0; tb < MB; ++tb) {
    acc[tb] = (v4i){0, 0, 0, 0};
    const int t = tb * 16 + r;
    const bool tok_ok = t < M;
    const int8_t* xrow = qx + (size_t)(tok_ok ? t : 0) * (size_t)K;
#pragma unroll
    for (int j = 0; j < kCH; ++j) {
      const int c = c0 + j;
      if (c < cs1) {  // uniform across the wavefront
        const int k = c * 64 + g * 16;
        v4i b = (v4i){0, 0, 0, 0};
        if (tok_ok && k < K) b = *reinterpret_cast<const v4i*>(xrow + k);
        acc[tb] = mfma_i8_16x16x64(a[j], b, acc[tb]);
      }
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
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) s_last = (atomicAdd(&counters[tile], 1) == splits - 1);
    __syncthreads();
    if (!s_last) return;
    __threadfence();
  }

  for (int e = threadIdx.x; e < elems; e += blockDim.x) {
    int32_t tot = 0;
    if (splits > 1) {
      const int32_t* base = partials + (size_t)tile * splits * elems + e;
      for (int sp = 0; sp < splits; ++sp) tot += __builtin_nontemporal_load(base + (size_t)sp * elems);
    } else {
      for (int w = 0; w < waves; ++w) tot += red[w * elems + e];
    }
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

}  // namespace

LinearPlan plan_linear(int64_t M, int64_t N, int64_t K) {
  LinearPlan p{};
  p.M = M;
  p.N = N;
  p.K = K;
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
  p.off_counters = off;
  if (p.splits > 1) off = align_up(off + (size_t)p.tiles * sizeof(int32_t), kWsAlign);
  p.off_partials = off;
  if (p.splits > 1)
    off = align_up(off + (size_t)p.tiles * p.splits * p.mb * 256 * sizeof(int32_t), kWsAlign);
  p.bytes = (M == 0 || N == 0) ? 0 : off;
  return p;
}

hipError_t launch_gemm(const LinearPlan& p, const int8_t* qx, const float* sx, const int8_t* wq,
                       const float* w_scale, uint16_t* y, int32_t* acc_out, int32_t* counters,
                       int32_t* partials, hipStream_t st) {
  const dim3 grid((unsigned)((int64_t)p.tiles * p.splits)), block(p.waves * kWave);
  const size_t lds = (size_t)p.waves * p.mb * 256 * sizeof(int32_t);
  const int M = (int)p.M, N = (int)p.N, K = (int)p.K;
#define QUASAR_GEMM_CASE(MB)                                                                    \
  case MB:                                                                                      \
    gemm_w8a8_kernel<MB><<<grid, block, lds, st>>>(qx, sx, wq, w_scale, M, N, K, p.splits,      \
                                                  p.chunks_per_split, y, acc_out, counters,     \
                                                  partials);                                    \
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
  return hipGetLastError();
}

}  // namespace quasar
