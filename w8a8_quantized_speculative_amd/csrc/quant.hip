// Row quantizers: offline weight preparation and the online activation step.
//
// Weights: w' = RN32(W * RN32(1/s)), one INT8 scale per output channel
// [Quasar, pt page §2 execution pipeline item 1; zh page §2 item 2].
// Activations: xs = RN32(X * s), one dynamic INT8 scale per token
// [pt page §2 item 2; nl page §2 pipeline "online"].
// Both are symmetric uniform quantizers [pt page §2].
//
// One workgroup of 256 threads owns one row.  Each thread handles 8-element
// units (16 bytes of bf16, 32 bytes of s); the row absmax is a wavefront
// max-reduction followed by a 4-entry LDS reduction.
#include "quasar_device.hpp"
#include "quasar_internal.hpp"

namespace quasar {
namespace {

constexpr int kRowThreads = 256;

template <bool kWeights>
__device__ __forceinline__ void load_unit(const uint16_t* __restrict__ row,
                                          const float* __restrict__ s, int64_t q, float v[8]) {
  const uint4 xv = *reinterpret_cast<const uint4*>(row + q * 8);
  const float4 s0 = *reinterpret_cast<const float4*>(s + q * 8);
  const float4 s1 = *reinterpret_cast<const float4*>(s + q * 8 + 4);
  float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t bits = (e & 1) ? (xw[e >> 1] >> 16) : (xw[e >> 1] & 0xffffu);
    // weights are divided by s (as a multiply by the rounded reciprocal),
    // activations multiplied by s
    const float f = kWeights ? 1.0f / sv[e] : sv[e];
    v[e] = bf16_to_f32(bits) * f;
  }
}

// Codes of 8-element unit q of a row: activations are stored row-major
// (row_base = row start), weights at their tile-packed position.
template <bool kWeights>
__device__ __forceinline__ void store_unit(int8_t* __restrict__ codes, float* __restrict__ xs_out,
                                           int64_t row, int64_t nch, int64_t q, const float v[8],
                                           float inv) {
  int c[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) c[e] = quant_code(v[e], inv);
  uint2 pk;
  pk.x = pack4_i8(c[0], c[1], c[2], c[3]);
  pk.y = pack4_i8(c[4], c[5], c[6], c[7]);
  *reinterpret_cast<uint2*>(codes + (kWeights ? packed_offset(row, q * 8, nch) : q * 8)) = pk;
  if (xs_out) {
    *reinterpret_cast<float4*>(xs_out + q * 8) = make_float4(v[0], v[1], v[2], v[3]);
    *reinterpret_cast<float4*>(xs_out + q * 8 + 4) = make_float4(v[4], v[5], v[6], v[7]);
  }
}

// K positions in [K, 64 * nch) of a packed weight row hold zero codes.
__device__ __forceinline__ void zero_k_padding(int8_t* __restrict__ wq, int64_t row, int64_t K,
                                               int64_t nch) {
  for (int64_t k = K + (int64_t)threadIdx.x * 16; k < nch * 64; k += kRowThreads * 16)
    *reinterpret_cast<uint4*>(wq + packed_offset(row, k, nch)) = make_uint4(0, 0, 0, 0);
}

// Row of the source matrix behind output row `row`.  In the gated order
// (gated_half = I > 0, the rows of a [gate; up] matrix of 2I rows), output rows
// 16 t .. 16 t + 7 are gate rows 8 t .. 8 t + 7 and 16 t + 8 .. 16 t + 15 are up
// rows 8 t .. 8 t + 7, so one 16-channel tile holds both factors of 8 outputs.
__device__ __forceinline__ int64_t source_row(int64_t row, int64_t gated_half) {
  if (gated_half == 0) return row;
  const int64_t t = row >> 4, i = row & 15;
  return (i < 8 ? 0 : gated_half) + t * 8 + (i & 7);
}

// Register-resident variant: the smoothed row stays in registers between the
// absmax pass and the quantize pass (K <= kUPT * 256 * 8).
template <bool kWeights, int kUPT>
__global__ __launch_bounds__(kRowThreads) void quantize_rows_reg_kernel(
    const uint16_t* __restrict__ src, const float* __restrict__ s, int64_t K,
    int8_t* __restrict__ codes, float* __restrict__ scales, float* __restrict__ xs_out,
    int64_t gated_half) {
  __shared__ float red[kRowThreads / kWave];
  const int64_t row = blockIdx.x;
  const int64_t units = K / 8;
  const uint16_t* xr = src + source_row(row, gated_half) * K;
  float v[kUPT][8];
  float amax = 0.0f;
#pragma unroll
  for (int u = 0; u < kUPT; ++u) {
    const int64_t q = (int64_t)u * kRowThreads + threadIdx.x;
    if (q < units) {
      load_unit<kWeights>(xr, s, q, v[u]);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[u][e]));
    }
  }
  amax = block_max(amax, red);
  const QParams qp = row_qparams(amax);
  const int64_t nch = (K + 63) / 64;
  int8_t* cr = kWeights ? codes : codes + row * K;
  float* xo = xs_out ? xs_out + row * K : nullptr;
#pragma unroll
  for (int u = 0; u < kUPT; ++u) {
    const int64_t q = (int64_t)u * kRowThreads + threadIdx.x;
    if (q < units) store_unit<kWeights>(cr, xo, row, nch, q, v[u], qp.inv);
  }
  if (kWeights) zero_k_padding(codes, row, K, nch);
  if (threadIdx.x == 0) scales[row] = qp.scale;
}

// Streaming variant for long rows: two passes over global memory.
template <bool kWeights>
__global__ __launch_bounds__(kRowThreads) void quantize_rows_stream_kernel(
    const uint16_t* __restrict__ src, const float* __restrict__ s, int64_t K,
    int8_t* __restrict__ codes, float* __restrict__ scales, float* __restrict__ xs_out,
    int64_t gated_half) {
  __shared__ float red[kRowThreads / kWave];
  const int64_t row = blockIdx.x;
  const int64_t units = K / 8;
  const uint16_t* xr = src + source_row(row, gated_half) * K;
  float amax = 0.0f;
  for (int64_t q = threadIdx.x; q < units; q += kRowThreads) {
    float v[8];
    load_unit<kWeights>(xr, s, q, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
  amax = block_max(amax, red);
  const QParams qp = row_qparams(amax);
  const int64_t nch = (K + 63) / 64;
  int8_t* cr = kWeights ? codes : codes + row * K;
  float* xo = xs_out ? xs_out + row * K : nullptr;
  for (int64_t q = threadIdx.x; q < units; q += kRowThreads) {
    float v[8];
    load_unit<kWeights>(xr, s, q, v);
    store_unit<kWeights>(cr, xo, row, nch, q, v, qp.inv);
  }
  if (kWeights) zero_k_padding(codes, row, K, nch);
  if (threadIdx.x == 0) scales[row] = qp.scale;
}

// Rows past N in the last 16-row tile of the packed weights hold zero codes.
__global__ __launch_bounds__(kRowThreads) void zero_pad_rows_kernel(int8_t* __restrict__ wq,
                                                                    int64_t N, int64_t nch) {
  const int64_t row = N + blockIdx.x;  // N <= row < 16 * tiles
  for (int64_t k = (int64_t)threadIdx.x * 16; k < nch * 64; k += kRowThreads * 16)
    *reinterpret_cast<uint4*>(wq + packed_offset(row, k, nch)) = make_uint4(0, 0, 0, 0);
}

// 4-bit weights [pt page §5, zh page §5: lower-bit verification as future
// work; read as the INT8 rule at qmax = 7]: code = clamp(rint(RN32(w' inv)),
// -7, 7) with inv = RN32(7 / absmax).  Two passes over the row (absmax, then
// codes); thread i packs the 8 positions 128 c + 8 j and 128 c + 64 + 8 j
// (j < 8) of pair unit i into 8 bytes of the 4-bit layout (w4_packed_offset).
__device__ __forceinline__ uint32_t w4_nibble(float v, float inv) {
  float r = __builtin_rintf(v * inv);
  r = fminf(fmaxf(r, -kQmaxW4), kQmaxW4);
  return (uint32_t)(int)r & 0xfu;
}

__global__ __launch_bounds__(kRowThreads) void quantize_rows_w4_kernel(
    const uint16_t* __restrict__ w, const float* __restrict__ s, int64_t K,
    int8_t* __restrict__ wq4, float* __restrict__ scales) {
  __shared__ float red[kRowThreads / kWave];
  const int64_t row = blockIdx.x;
  const uint16_t* wr = w + row * K;
  const int64_t units = K / 8;
  float amax = 0.0f;
  for (int64_t q = threadIdx.x; q < units; q += kRowThreads) {
    float v[8];
    load_unit<true>(wr, s, q, v);
#pragma unroll
    for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
  }
  amax = block_max(amax, red);
  const QParams qp = row_qparams(amax, kQmaxW4);
  const int64_t ncp = K / 128;
  for (int64_t p = threadIdx.x; p < K / 16; p += kRowThreads) {
    const int64_t qlo = (p >> 3) * 16 + (p & 7);  // unit of the chunk-2c half
    float lo[8], hi[8];
    load_unit<true>(wr, s, qlo, lo);
    load_unit<true>(wr, s, qlo + 8, hi);  // 64 positions on: chunk 2c + 1
    uint32_t by[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) by[e] = w4_nibble(lo[e], qp.inv) | (w4_nibble(hi[e], qp.inv) << 4);
    uint2 pk;
    pk.x = by[0] | (by[1] << 8) | (by[2] << 16) | (by[3] << 24);
    pk.y = by[4] | (by[5] << 8) | (by[6] << 16) | (by[7] << 24);
    *reinterpret_cast<uint2*>(wq4 + w4_packed_offset(row, qlo * 8, ncp)) = pk;
  }
  if (threadIdx.x == 0) scales[row] = qp.scale;
}

// Rows past N in the last tile of the 4-bit layout hold zero codes.
__global__ __launch_bounds__(kRowThreads) void zero_pad_rows_w4_kernel(int8_t* __restrict__ wq4,
                                                                       int64_t N, int64_t ncp) {
  const int64_t row = N + blockIdx.x;  // N <= row < 16 * tiles
  for (int64_t i = threadIdx.x; i < ncp * 4; i += kRowThreads)  // 16 bytes per (pair, K group)
    *reinterpret_cast<uint4*>(wq4 + w4_packed_offset(row, (i >> 2) * 128 + (i & 3) * 16, ncp)) =
        make_uint4(0, 0, 0, 0);
}

template <bool kWeights>
hipError_t launch_rows(const uint16_t* src, const float* s, int64_t rows, int64_t K, int8_t* codes,
                       float* scales, float* xs_out, hipStream_t st, int64_t gated_half = 0) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((unsigned)rows), block(kRowThreads);
  const int64_t upt = (K / 8 + kRowThreads - 1) / kRowThreads;
  if (upt <= 1)
    quantize_rows_reg_kernel<kWeights, 1><<<grid, block, 0, st>>>(src, s, K, codes, scales, xs_out,
                                                               gated_half);
  else if (upt <= 2)
    quantize_rows_reg_kernel<kWeights, 2><<<grid, block, 0, st>>>(src, s, K, codes, scales, xs_out,
                                                               gated_half);
  else if (upt <= 4)
    quantize_rows_reg_kernel<kWeights, 4><<<grid, block, 0, st>>>(src, s, K, codes, scales, xs_out,
                                                               gated_half);
  else if (upt <= 8)
    quantize_rows_reg_kernel<kWeights, 8><<<grid, block, 0, st>>>(src, s, K, codes, scales, xs_out,
                                                               gated_half);
  else
    quantize_rows_stream_kernel<kWeights><<<grid, block, 0, st>>>(src, s, K, codes, scales, xs_out,
                                                               gated_half);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_weights(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                   int8_t* wq, float* w_scale, hipStream_t st, bool gated) {
  hipError_t e = launch_rows<true>(w, s, N, K, wq, w_scale, nullptr, st, gated ? N / 2 : 0);
  const int64_t pad_rows = (N + 15) / 16 * 16 - N;
  if (e != hipSuccess || pad_rows == 0) return e;
  zero_pad_rows_kernel<<<dim3((unsigned)pad_rows), dim3(kRowThreads), 0, st>>>(wq, N, (K + 63) / 64);
  return hipGetLastError();
}

hipError_t launch_quantize_weights_w4(const uint16_t* w, const float* s, int64_t N, int64_t K,
                                      int8_t* wq4, float* w_scale, hipStream_t st) {
  if (N == 0) return hipSuccess;
  quantize_rows_w4_kernel<<<dim3((unsigned)N), dim3(kRowThreads), 0, st>>>(w, s, K, wq4, w_scale);
  hipError_t e = hipGetLastError();
  const int64_t pad_rows = (N + 15) / 16 * 16 - N;
  if (e != hipSuccess || pad_rows == 0) return e;
  zero_pad_rows_w4_kernel<<<dim3((unsigned)pad_rows), dim3(kRowThreads), 0, st>>>(wq4, N, K / 128);
  return hipGetLastError();
}

hipError_t launch_quantize_activations(const uint16_t* x, const float* s, int64_t M, int64_t K,
                                       int8_t* qx, float* sx, float* xs_out, hipStream_t st) {
  return launch_rows<false>(x, s, M, K, qx, sx, xs_out, st);
}

}  // namespace quasar
