// Device-side building blocks shared by the gfx950 kernels of libquasar.
//
// Everything here is binary32 arithmetic with one rounding per operation: the
// library is compiled with -ffp-contract=off, so no multiply-add is fused, and
// fp32 division is the correctly rounded default of hipcc.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quasar {

typedef int v4i __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;    // CDNA wavefront width
constexpr float kQmax = 127.0f;

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}

// Round-to-nearest-even binary32 -> bfloat16 for finite inputs (the path never
// produces NaN): add 0x7FFF plus the lowest kept bit, drop the low half.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Per-row symmetric INT8 parameters from a row's absolute maximum:
// scale = RN32(A / 127), inv = RN32(127 / A); an all-zero row gets 0 and 0.
struct QParams {
  float scale;
  float inv;
};

__device__ __forceinline__ QParams row_qparams(float amax, float qmax = kQmax) {
  QParams p;
  if (amax == 0.0f) {
    p.scale = 0.0f;
    p.inv = 0.0f;
  } else {
    p.scale = amax / qmax;
    p.inv = qmax / amax;
  }
  return p;
}

// code = clamp(rint(RN32(v * inv)), -127, 127), rint rounding half to even.
__device__ __forceinline__ int quant_code(float v, float inv) {
  float r = __builtin_rintf(v * inv);
  r = fminf(fmaxf(r, -kQmax), kQmax);
  return (int)r;
}

// The same code without the clamp, for |v| <= A and inv = RN32(127 / A): then
// |v * inv| <= 127 * (1 + 2^-24), whose binary32 rounding is at most 127 + 2^-17,
// and rint of that is 127, so the clamp can never act.
__device__ __forceinline__ int quant_code_in_range(float v, float inv) {
  return (int)__builtin_rintf(v * inv);
}

// The same code as the low byte of a binary32 encoding: for |q| <= 127 + 2^-17
// (q = RN32(v * inv) as above), q + 1.5 * 2^23 lies in [2^23, 2^24), where
// consecutive binary32 values are 1 apart, so the addition's round-to-nearest-
// even result is exactly 1.5 * 2^23 + rint(q).  Its encoding is 0x4B400000 +
// rint(q), whose low 8 bits are rint(q) in two's complement.  Two operations
// per code instead of a round, a convert and a mask.
__device__ __forceinline__ uint32_t quant_code_biased(float v, float inv) {
  const float q = v * inv;
  return __float_as_uint(q + 12582912.0f);
}

// Bytes 0 of four words into one word (byte i from word i).
__device__ __forceinline__ uint32_t pack4_low_bytes(uint32_t a, uint32_t b, uint32_t c,
                                                    uint32_t d) {
  return (a & 0xffu) | ((b & 0xffu) << 8) | ((c & 0xffu) << 16) | (d << 24);
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)(d & 0xff) << 24);
}

// Max over the 64 lanes of a wavefront (all lanes receive the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
  return v;
}

// Max over the 64 lanes of a wavefront for NON-NEGATIVE floats, on their bit
// patterns (which order like unsigned integers), with DPP row operations
// instead of LDS permutes: butterflies within each row of 16 lanes, then the
// row broadcasts carry the maxima to lane 63, which is read back as a scalar.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ uint32_t dpp_umax(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, kCtrl, kRowMask, 0xf, false);
  return v > o ? v : o;
}

__device__ __forceinline__ float wave_max_nonneg(float f) {
  uint32_t v = __float_as_uint(f);
  v = dpp_umax<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_umax<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]
  v = dpp_umax<0x141, 0xf>(v);  // row_half_mirror
  v = dpp_umax<0x140, 0xf>(v);  // row_mirror: every lane holds its row's max
  v = dpp_umax<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_umax<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3: lane 63 has the max
  return __uint_as_float((uint32_t)__builtin_amdgcn_readlane((int)v, 63));
}

// Tile-packed INT8 weight layout.  The weights are stored in the exact order
// the MFMA A operand is loaded: for each 16-row tile t and 64-wide K chunk c, a
// 1 KB block holds lane l's 16 bytes at l*16, where lane l = 16*g + r carries
// row 16t + r, K positions 64c + 16g .. 64c + 16g + 15.  A wavefront thus reads
// one chunk of one tile as a single contiguous 1 KB.  Rows past N and K past K
// are zero padding.
__host__ __device__ __forceinline__ int64_t packed_offset(int64_t n, int64_t k, int64_t nch) {
  const int64_t t = n >> 4, r = n & 15, c = k >> 6, g = (k >> 4) & 3, b = k & 15;
  return ((t * nch + c) * 64 + g * 16 + r) * 16 + b;
}

// 4-bit weight layout (the INT4 verifier variant): the codes (two's complement
// nibbles) of 64-wide chunks 2c and 2c + 1 of a tile share one 1 KB block, the
// chunk 2c code in the low nibble and the chunk 2c + 1 code in the high nibble
// of the byte the INT8 layout gives K position 64 (2c) + j.  So one 16-byte
// load per lane carries the A operands of two chunks: (v << 4) & 0xF0F0F0F0
// and v & 0xF0F0F0F0 are the chunks' codes times 16, as int8 bytes.
// k must lie in the low half of its 128-block (k % 128 < 64); ncp = K / 128.
__host__ __device__ __forceinline__ int64_t w4_packed_offset(int64_t n, int64_t k, int64_t ncp) {
  const int64_t t = n >> 4, r = n & 15, cp = k >> 7, g = (k >> 4) & 3, b = k & 15;
  return ((t * ncp + cp) * 64 + g * 16 + r) * 16 + b;
}
constexpr float kQmaxW4 = 7.0f;  // 4-bit weight codes in [-7, 7]

// Block-wide max; `red` must hold blockDim.x / 64 floats.  Ends with a barrier
// so `red` can be reused afterwards.
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int nw = blockDim.x / kWave;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

// v_mfma_i32_16x16x64_i8: D[16x16] += A[16x64] * B[64x16], int8 operands, int32
// accumulators.  Lane l holds row (l % 16) of A and column (l % 16) of B, each as
// 16 consecutive K positions of one K-group (l / 16); the hardware pairs the
// same byte of A and B, so any consistent K order gives the same dot products.
// Result: lane l, register r holds D[4 * (l / 16) + r][l % 16].
__device__ __forceinline__ v4i mfma_i8_16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Raw buffer resource (stride 0): loads at byte offsets >= num_bytes return
// zero without touching memory.  Word 3 selects 32-bit untyped data, as the
// gfx9 family expects for raw buffer access.
typedef __amdgpu_buffer_rsrc_t buffer_rsrc;
constexpr int kOutOfRange = 0x7ffffff0;  // an offset past every resource this library builds
constexpr int kNonTemporal = 2;          // cache-policy bit: streaming (nt) access

__device__ __forceinline__ buffer_rsrc make_rsrc(const void* base, uint32_t num_bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)num_bytes,
                                           0x00020000);
}

template <int kAux = 0>
__device__ __forceinline__ int load4(buffer_rsrc rs, int offset) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, offset, 0, kAux);
}

template <int kAux = 0>
__device__ __forceinline__ v4i load16(buffer_rsrc rs, int offset) {
  return __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(rs, offset, 0, kAux));
}

}  // namespace quasar
