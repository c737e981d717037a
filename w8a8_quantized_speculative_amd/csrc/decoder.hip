// The non-linear steps of a Qwen3-8B-shaped decoder around the W8A8 linears,
// for a synthetic full verify step [Quasar, pt page §2 execution pipeline:
// the verifier runs the target model over the drafted positions in one pass;
// zh page §2].  They are not part of the quantized linear; they exist so that
// the linears' share of a whole verify step can be measured with every
// dependency between them in place.
//
// Arithmetic is binary32 with one rounding per operation (the library is
// built with -ffp-contract=off); every tensor that leaves a kernel is BF16
// (round to nearest even) except the residual stream, which stays binary32.
//
// Kernels:
//   embed_kernel         h[m, :] = E[tok[m], :]
//   rmsnorm_kernel       (h += delta), out = BF16(h * rsqrt(mean(h^2) + eps) * gamma)
//   qk_rope_cache_kernel per-head RMSNorm of q and k, rotate-half RoPE, k and v
//                        appended to the cache, q written for the attention
//   attn_chunk_mfma_kernel  one KV head x 64 cached positions: partial softmax
//                        (max, sum of exp, unnormalised output) of the group's
//                        query rows, both products on the matrix cores (groups
//                        of at most 32 query rows)
//   attn_chunk_kernel    the same on the vector ALUs, for wider groups
//   attn_combine_kernel  merges the chunks of a query row
//   silu_mul_kernel      out = BF16(silu(gate) * up) over the gate_up output
#include "quasar_device.hpp"
#include "quasar_internal.hpp"

namespace quasar {
namespace {

constexpr int kNormThreads = 256;

// Sum over a block (blockDim.x threads, a multiple of 64); `red` holds
// blockDim.x / 64 floats.  Ends with a barrier so `red` can be reused.
__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int nw = blockDim.x / kWave;
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < nw; ++w) r += red[w];
  __syncthreads();
  return r;
}

__global__ __launch_bounds__(kNormThreads) void embed_kernel(const int32_t* __restrict__ tok,
                                                             const uint16_t* __restrict__ table,
                                                             int V, int H, float* __restrict__ h) {
  const int m = blockIdx.x;
  const int t = tok[m];
  const bool ok = t >= 0 && t < V;
  const uint16_t* row = table + (size_t)(ok ? t : 0) * H;
  for (int j = threadIdx.x; j < H; j += blockDim.x)
    h[(size_t)m * H + j] = ok ? bf16_to_f32(row[j]) : 0.0f;
}

// One block per row.  mean(h^2) is a binary32 sum of squares, per thread in
// index order, then across the block.  Rows of up to 16 values per thread
// (H % 4 == 0) stay in registers between the two passes, loaded 4 at a time.
constexpr int kNormPerThread = 16;

__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(float* __restrict__ h,
                                                               const uint16_t* __restrict__ delta,
                                                               const float* __restrict__ gamma,
                                                               int H, float eps,
                                                               uint16_t* __restrict__ out) {
  __shared__ float red[kNormThreads / kWave];
  const int m = blockIdx.x, tid = threadIdx.x;
  float* hr = h + (size_t)m * H;
  const uint16_t* dr = delta ? delta + (size_t)m * H : nullptr;
  uint16_t* orow = out + (size_t)m * H;
  if ((H & 3) == 0 && H <= kNormThreads * kNormPerThread) {
    // 4 values per 16-byte load, every load of the row issued before the
    // first use (the rows and gamma are 16-byte aligned, the BF16 rows 8)
    constexpr int kVec = kNormPerThread / 4;
    float4 v[kVec];
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const int j = (tid + k * kNormThreads) * 4;
      const float4 x = *reinterpret_cast<const float4*>(hr + (j < H ? j : 0));
      v[k] = j < H ? x : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
    if (dr) {
      uint2 dv[kVec];
#pragma unroll
      for (int k = 0; k < kVec; ++k) {
        const int j = (tid + k * kNormThreads) * 4;
        dv[k] = *reinterpret_cast<const uint2*>(dr + (j < H ? j : 0));
      }
#pragma unroll
      for (int k = 0; k < kVec; ++k) {
        if ((tid + k * kNormThreads) * 4 < H) {
          v[k].x = v[k].x + bf16_to_f32(dv[k].x & 0xffffu);
          v[k].y = v[k].y + bf16_to_f32(dv[k].x >> 16);
          v[k].z = v[k].z + bf16_to_f32(dv[k].y & 0xffffu);
          v[k].w = v[k].w + bf16_to_f32(dv[k].y >> 16);
        }
      }
    }
    float ss = 0.0f;
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      ss = ss + v[k].x * v[k].x;
      ss = ss + v[k].y * v[k].y;
      ss = ss + v[k].z * v[k].z;
      ss = ss + v[k].w * v[k].w;
    }
    const float tot = block_sum(ss, red);
    const float r = 1.0f / sqrtf(tot / (float)H + eps);
#pragma unroll
    for (int k = 0; k < kVec; ++k) {
      const int j = (tid + k * kNormThreads) * 4;
      if (j < H) {
        if (dr) *reinterpret_cast<float4*>(hr + j) = v[k];
        const float4 gm = *reinterpret_cast<const float4*>(gamma + j);
        uint2 o;
        o.x = f32_to_bf16_rne(v[k].x * r * gm.x) | (f32_to_bf16_rne(v[k].y * r * gm.y) << 16);
        o.y = f32_to_bf16_rne(v[k].z * r * gm.z) | (f32_to_bf16_rne(v[k].w * r * gm.w) << 16);
        *reinterpret_cast<uint2*>(orow + j) = o;
      }
    }
    return;
  }
  // wider rows: the residual add first, then the two passes over memory
  float ss = 0.0f;
  for (int j = tid; j < H; j += kNormThreads) {
    float v = hr[j];
    if (dr) {
      v = v + bf16_to_f32(dr[j]);
      hr[j] = v;
    }
    ss = ss + v * v;
  }
  const float tot = block_sum(ss, red);
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  for (int j = tid; j < H; j += kNormThreads)
    orow[j] = (uint16_t)f32_to_bf16_rne(hr[j] * r * gamma[j]);
}

// One block of D threads per (token, head of q, k or v).  Token m = b T + i sits
// at position pos0 + i.
__global__ void qk_rope_cache_kernel(const uint16_t* __restrict__ qkv, const float* __restrict__ q_gamma,
                                     const float* __restrict__ k_gamma, int T, int Hq, int Hkv,
                                     int D, int pos0, int Lmax, double log2_base, float eps,
                                     uint16_t* __restrict__ q_out, uint16_t* __restrict__ k_cache,
                                     uint16_t* __restrict__ v_cache) {
  __shared__ float red[4];
  __shared__ float xs[256];
  const int m = blockIdx.x, head = blockIdx.y, d = threadIdx.x;
  const int b = m / T, i = m - b * T, pos = pos0 + i;
  const int W = (Hq + 2 * Hkv) * D;
  const float x = bf16_to_f32(qkv[(size_t)m * W + (size_t)head * D + d]);
  if (head >= Hq + Hkv) {  // v: copied to the cache
    const int g = head - Hq - Hkv;
    v_cache[(((size_t)b * Hkv + g) * Lmax + pos) * D + d] = qkv[(size_t)m * W + (size_t)head * D + d];
    return;
  }
  const bool is_q = head < Hq;
  const float tot = block_sum(x * x, red);
  const float r = 1.0f / sqrtf(tot / (float)D + eps);
  const float y = x * r * (is_q ? q_gamma[d] : k_gamma[d]);
  xs[d] = y;
  __syncthreads();
  // rotate half: pair (j, j + D/2) turns by pos * base^(-2j / D).  The angle
  // and its reduction to [0, 2 pi) are binary64: in binary32 the rounding of
  // the exponent alone moves base^(-2j/D) by ~1e-6 relative, ~1e-3 rad at
  // position 2047; reduced in binary64 the angle is within ~2.4e-7 rad.
  const int half = D / 2, j = d < half ? d : d - half;
  const double two_pi = 6.283185307179586476925;
  const double inv_freq = exp2(-(double)(2 * j) / (double)D * log2_base);
  double ang = (double)pos * inv_freq;
  ang = ang - floor(ang / two_pi) * two_pi;
  const float c = cosf((float)ang), s = sinf((float)ang);
  const float o = d < half ? y * c - xs[d + half] * s : y * c + xs[d - half] * s;
  const uint16_t ob = (uint16_t)f32_to_bf16_rne(o);
  if (is_q) {
    q_out[(size_t)m * Hq * D + (size_t)head * D + d] = ob;
  } else {
    const int g = head - Hq;
    k_cache[(((size_t)b * Hkv + g) * Lmax + pos) * D + d] = ob;
  }
}

// Attention partials.  Block (chunk c, kv head g, sequence b): the R = (Hq / Hkv) T
// query rows of the group (row r = head-in-group * T + i) against cached
// positions [64 c, 64 c + 64), causal: query i sees positions < pos0 + i + 1.
// Scores are binary32 dot products in d order, scaled by 1/sqrt(D).
//
// Layout: the chunk's keys go to LDS transposed in BF16 pairs, kT2[d/2][t] =
// (K[t][d], K[t][d+1]) (rows padded to 65 words against bank conflicts on the
// transposing writes), so lane t of a wavefront reads two of key t's values
// per 32-bit access; values stay row-major as pairs, vs2[t][d/2], and so do the
// query rows, qs2[r][d/2], read as 4-byte broadcasts (a 16-byte binary32
// broadcast moves four times the bytes through the LDS crossbar, and scalar
// loads of the rows from memory were slower still).  Wavefront w of 8 owns
// rows w, w + 8, ...: it takes them four at a time through scores (lane =
// key), softmax (wavefront reductions) and P V (lane = a pair of d), so after
// the one barrier no wavefront waits for another.  The loops run over the whole chunk (keys
// past the window carry p = 0 and zero values).
constexpr int kAttnChunk = 64;
constexpr int kAttnThreads = 512;
constexpr int kAttnKTStride = kAttnChunk + 1;  // words per kT2 row
constexpr int kAttnMaxRows = 64;  // (Hq / Hkv) * T
constexpr int kAttnD = 128;
constexpr int kAttnRowGroup = 4;

__host__ __device__ constexpr int attn_lds_bytes(int R) {
  return (kAttnD / 2) * kAttnKTStride * 4 + kAttnChunk * kAttnD * 2 + R * kAttnD * 2 +
         R * kAttnChunk * 4;
}

__global__ __launch_bounds__(kAttnThreads) void attn_chunk_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, int T, int Hq, int Hkv, int pos0, int Lmax,
    int nchunks, float scale, float* __restrict__ pm, float* __restrict__ pl,
    float* __restrict__ po) {
  extern __shared__ __align__(16) char smem[];
  const int c = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv, R = G * T;
  const int klen = pos0 + T;  // keys after this step's append
  const int t0 = c * kAttnChunk;
  const int nt = min(kAttnChunk, klen - t0);
  uint32_t* kT2 = reinterpret_cast<uint32_t*>(smem);                       // [D/2][65]
  uint32_t* vs2 = kT2 + (kAttnD / 2) * kAttnKTStride;                      // [64][D/2]
  uint32_t* qs2 = vs2 + kAttnChunk * (kAttnD / 2);                         // [R][D/2]
  float* ps = reinterpret_cast<float*>(qs2 + R * (kAttnD / 2));             // [R][64]
  const int tid = threadIdx.x;

  // the chunk's keys and values (buffer resources: reads past its nt keys
  // return zero, with no branch), 16 bytes = 8 values per load
  const size_t kv0 = (((size_t)b * Hkv + g) * Lmax + t0) * kAttnD;
  const buffer_rsrc krs = make_rsrc(k_cache + kv0, (uint32_t)nt * kAttnD * 2u);
  const buffer_rsrc vrs = make_rsrc(v_cache + kv0, (uint32_t)nt * kAttnD * 2u);
  const buffer_rsrc qrs = make_rsrc(q + (size_t)b * T * Hq * kAttnD, (uint32_t)(T * Hq * kAttnD * 2));
  v4i kreg[2], vreg[2], qreg[2];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = tid + kAttnThreads * k;  // 1024 units of a 64 x 128 chunk
    const int t = u >> 4, d0 = (u & 15) * 8;
    kreg[k] = load16(krs, (t * kAttnD + d0) * 2);
    vreg[k] = load16(vrs, (t * kAttnD + d0) * 2);
    const int r = u >> 4;  // query row r (of R <= 64), 8 values at d0
    const int hh = r / T, i = r - hh * T;
    qreg[k] = load16(qrs, r < R ? ((i * Hq + g * G + hh) * kAttnD + d0) * 2 : kOutOfRange);
  }
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int u = tid + kAttnThreads * k;
    const int t = u >> 4, d0 = (u & 15) * 8;
    kT2[(d0 / 2 + 0) * kAttnKTStride + t] = (uint32_t)kreg[k].x;
    kT2[(d0 / 2 + 1) * kAttnKTStride + t] = (uint32_t)kreg[k].y;
    kT2[(d0 / 2 + 2) * kAttnKTStride + t] = (uint32_t)kreg[k].z;
    kT2[(d0 / 2 + 3) * kAttnKTStride + t] = (uint32_t)kreg[k].w;
    *reinterpret_cast<v4i*>(vs2 + t * (kAttnD / 2) + d0 / 2) = vreg[k];
    if (t < R) *reinterpret_cast<v4i*>(qs2 + t * (kAttnD / 2) + d0 / 2) = qreg[k];
  }
  __syncthreads();

  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  for (int r0 = wave; r0 < R; r0 += kAttnRowGroup * (kAttnThreads / kWave)) {
    // rows past R are computed on row R - 1 and dropped: no branch inside the
    // loops, so the scheduler can issue LDS reads iterations ahead
    int rows[kAttnRowGroup], rc[kAttnRowGroup];
#pragma unroll
    for (int j = 0; j < kAttnRowGroup; ++j) {
      rows[j] = r0 + j * (kAttnThreads / kWave);
      rc[j] = rows[j] < R ? rows[j] : R - 1;
    }
    // scores: lane = key
    float acc[kAttnRowGroup] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
    for (int dp = 0; dp < kAttnD / 2; ++dp) {
      const uint32_t kw = kT2[dp * kAttnKTStride + lane];
      const float k0 = bf16_to_f32(kw & 0xffffu), k1 = bf16_to_f32(kw >> 16);
#pragma unroll
      for (int j = 0; j < kAttnRowGroup; ++j) {
        const uint32_t qw = qs2[rc[j] * (kAttnD / 2) + dp];
        acc[j] = acc[j] + bf16_to_f32(qw & 0xffffu) * k0;
        acc[j] = acc[j] + bf16_to_f32(qw >> 16) * k1;
      }
    }
    // softmax pieces of each row
#pragma unroll
    for (int j = 0; j < kAttnRowGroup; ++j) {
      const int r = rows[j];
      if (r >= R) continue;
      const int i = r % T;
      const bool valid = lane < nt && t0 + lane <= pos0 + i;
      const float sc = valid ? acc[j] * scale : -INFINITY;
      const float mx = wave_max(sc);
      const float p = mx == -INFINITY ? 0.0f : expf(sc - mx);
      float sum = p;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
      ps[r * kAttnChunk + lane] = p;
      if (lane == 0) {
        const size_t pi = (((size_t)b * Hq + g * G + r / T) * T + i) * nchunks + c;
        pm[pi] = mx;
        pl[pi] = sum;
      }
    }
    // this wavefront's own p rows are read back below: LDS executes a
    // wavefront's accesses in order; keep the compiler from reordering
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // P V: lane = d pair (2 lane, 2 lane + 1), keys in order, 4 per step
    float o[kAttnRowGroup][2] = {};
#pragma unroll 4
    for (int t = 0; t < kAttnChunk; t += 4) {
      uint32_t vw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) vw[e] = vs2[(t + e) * (kAttnD / 2) + lane];
#pragma unroll
      for (int j = 0; j < kAttnRowGroup; ++j) {
        const float4 p4 = *reinterpret_cast<const float4*>(ps + rc[j] * kAttnChunk + t);
        const float pe[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[j][0] = o[j][0] + pe[e] * bf16_to_f32(vw[e] & 0xffffu);
          o[j][1] = o[j][1] + pe[e] * bf16_to_f32(vw[e] >> 16);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kAttnRowGroup; ++j) {
      const int r = rows[j];
      if (r >= R) continue;
      const size_t pi = (((size_t)b * Hq + g * G + r / T) * T + r % T) * nchunks + c;
      *reinterpret_cast<float2*>(po + pi * kAttnD + 2 * lane) = make_float2(o[j][0], o[j][1]);
    }
  }
}

// Wavefront max and sum by DPP row operations (no LDS permutes): butterflies
// within rows of 16 lanes, then row broadcasts carry the totals to lane 63,
// read back as a scalar.  For the sum, lanes outside a broadcast's row mask
// add zero.
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_fmax(float v) {
  const float o = __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v),
                                                             kCtrl, kRowMask, 0xf, false));
  return fmaxf(v, o);
}
template <int kCtrl, int kRowMask>
__device__ __forceinline__ float dpp_fadd(float v) {
  const float o = __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), kCtrl, kRowMask,
                                                             0xf, false));
  return v + o;
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = dpp_fmax<0xB1, 0xf>(v);   // quad_perm [1,0,3,2]
  v = dpp_fmax<0x4E, 0xf>(v);   // quad_perm [2,3,0,1]
  v = dpp_fmax<0x141, 0xf>(v);  // row_half_mirror
  v = dpp_fmax<0x140, 0xf>(v);  // row_mirror
  v = dpp_fmax<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_fmax<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_fadd<0xB1, 0xf>(v);
  v = dpp_fadd<0x4E, 0xf>(v);
  v = dpp_fadd<0x141, 0xf>(v);
  v = dpp_fadd<0x140, 0xf>(v);
  v = dpp_fadd<0x142, 0xa>(v);
  v = dpp_fadd<0x143, 0xc>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// The same partials on the matrix cores, for groups of at most 32 query rows
// (the Qwen3-8B window: 4 heads per KV head x 6 positions = 24).  Eight
// wavefronts:
//   scores  wavefront w computes the 16 x 16 tile (row tile w / 4, key tile
//           w % 4) of Q K^T with four v_mfma_f32_16x16x32_bf16 over D = 128,
//           its operands read straight from memory (16 contiguous bytes of a
//           q row and of a key row per lane); products of BF16 values are
//           exact in binary32;
//   softmax per row over the 64 keys in LDS (lane = key);
//   P V     wavefront w owns output dimensions 16 w .. 16 w + 15 of both row
//           tiles: sixteen v_mfma_f32_16x16x4_f32 over the keys, P in binary32
//           (not rounded to BF16), V from LDS.
// Operand layout of both MFMAs: lane l supplies row (or column) l % 16 at the
// k positions of group l / 16; result register j of lane l is row
// 4 (l / 16) + j, column l % 16.
constexpr int kMfmaRows = 32;
constexpr int kAttnResidentWgs = 1024;  // chunk workgroups resident at once: ~4 per CU on 256 CUs
constexpr int kSsStride = kAttnChunk + 1;  // floats per score row in LDS
constexpr int kVsStride = kAttnD + 8;      // BF16 per value row in LDS

typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kAttnThreads) void attn_chunk_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, int T, int Hq, int Hkv, int pos0, int Lmax, int nparts,
    int cpw, float scale, float* __restrict__ pm, float* __restrict__ pl, float* __restrict__ po) {
  __shared__ float ss[kMfmaRows * kSsStride];
  __shared__ float sfac[kMfmaRows];  // per-row rescale of the running output, this chunk
  __shared__ __align__(16) uint16_t vs[kAttnChunk * kVsStride];
  const int part = blockIdx.x, g = blockIdx.y, b = blockIdx.z;
  const int G = Hq / Hkv, R = G * T;
  const int klen = pos0 + T;
  const int nch = (klen + kAttnChunk - 1) / kAttnChunk;
  const int c_begin = part * cpw, c_end = min(c_begin + cpw, nch);
  const int tid = threadIdx.x, lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int rl = lane & 15, grp = lane >> 4;

  // this wavefront's q operands, once for all of the workgroup's chunks
  const buffer_rsrc qrs = make_rsrc(q + (size_t)b * T * Hq * kAttnD, (uint32_t)(T * Hq * kAttnD * 2));
  const int rt = wave >> 2, kt = wave & 3;
  const int qr = rt * 16 + rl;  // A row: query row of the group
  const int qhh = qr / T, qi = qr - qhh * T;
  const int qbase = qr < R ? (qi * Hq + g * G + qhh) * kAttnD * 2 : kOutOfRange;
  const int kkey = kt * 16 + rl;  // B column: key of the chunk
  v4i qa[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qa[kk] = load16(qrs, qr < R ? qbase + (kk * 32 + grp * 8) * 2 : kOutOfRange);

  // running softmax of the rows this wavefront owns (rows wave + 8 jr), and the
  // running unnormalised output of its 16 dimensions for both row tiles
  constexpr int kRowsPerWave = kMfmaRows / (kAttnThreads / kWave);
  float m_run[kRowsPerWave], l_run[kRowsPerWave];
#pragma unroll
  for (int jr = 0; jr < kRowsPerWave; ++jr) {
    m_run[jr] = -INFINITY;
    l_run[jr] = 0.0f;
  }
  const int dcol = wave * 16 + rl;
  v4f o[kMfmaRows / 16] = {};

  for (int c = c_begin; c < c_end; ++c) {
    const int t0 = c * kAttnChunk;
    const int nt = min(kAttnChunk, klen - t0);
    const size_t kv0 = (((size_t)b * Hkv + g) * Lmax + t0) * kAttnD;
    const buffer_rsrc krs = make_rsrc(k_cache + kv0, (uint32_t)nt * kAttnD * 2u);
    const buffer_rsrc vrs = make_rsrc(v_cache + kv0, (uint32_t)nt * kAttnD * 2u);
    v4i vreg[2], kb[4];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = tid + kAttnThreads * k;
      vreg[k] = load16(vrs, ((u >> 4) * kAttnD + (u & 15) * 8) * 2);
    }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) kb[kk] = load16(krs, (kkey * kAttnD + kk * 32 + grp * 8) * 2);
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
      acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf16, qa[kk]),
                                                    __builtin_bit_cast(v8bf16, kb[kk]), acc, 0, 0,
                                                    0);
    __syncthreads();  // the previous chunk's P V reads of ss and vs are done
    // scaled, masked scores and the value chunk into LDS
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = rt * 16 + grp * 4 + j;
      const int i = row % T;
      const bool valid = row < R && kkey < nt && t0 + kkey <= pos0 + i;
      ss[row * kSsStride + kkey] = valid ? acc[j] * scale : -INFINITY;
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int u = tid + kAttnThreads * k;
      *reinterpret_cast<v4i*>(vs + (u >> 4) * kVsStride + (u & 15) * 8) = vreg[k];
    }
    __syncthreads();
    // softmax pieces, lane = key, folded into the running maximum and sum
#pragma unroll
    for (int jr = 0; jr < kRowsPerWave; ++jr) {
      const int row = wave + jr * (kAttnThreads / kWave);
      if (row >= R) continue;
      const float sc = ss[row * kSsStride + lane];
      const float new_m = fmaxf(m_run[jr], wave_max_dpp(sc));
      const float fac = m_run[jr] == -INFINITY ? 0.0f : expf(m_run[jr] - new_m);
      const float p = new_m == -INFINITY ? 0.0f : expf(sc - new_m);
      l_run[jr] = l_run[jr] * fac + wave_sum_dpp(p);
      m_run[jr] = new_m;
      ss[row * kSsStride + lane] = p;
      if (lane == 0) sfac[row] = fac;
    }
    __syncthreads();
    // P V: rescale the running output rows, then add this chunk's keys; the two
    // row tiles' MFMA chains interleave and share each value read
#pragma unroll
    for (int rt2 = 0; rt2 < kMfmaRows / 16; ++rt2)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int row = rt2 * 16 + grp * 4 + j;
        o[rt2][j] = o[rt2][j] * (row < R ? sfac[row] : 0.0f);
      }
#pragma unroll
    for (int kk = 0; kk < kAttnChunk / 4; ++kk) {
      const int key = kk * 4 + grp;
      const float vb = bf16_to_f32(vs[key * kVsStride + dcol]);
#pragma unroll
      for (int rt2 = 0; rt2 < kMfmaRows / 16; ++rt2) {
        const int prow = rt2 * 16 + rl;
        const float pa = prow < R ? ss[prow * kSsStride + key] : 0.0f;
        o[rt2] = __builtin_amdgcn_mfma_f32_16x16x4f32(pa, vb, o[rt2], 0, 0, 0);
      }
    }
  }
  // the workgroup's partials
#pragma unroll
  for (int jr = 0; jr < kRowsPerWave; ++jr) {
    const int row = wave + jr * (kAttnThreads / kWave);
    if (row < R && lane == 0) {
      const size_t pi = (((size_t)b * Hq + g * G + row / T) * T + row % T) * nparts + part;
      pm[pi] = m_run[jr];
      pl[pi] = l_run[jr];
    }
  }
#pragma unroll
  for (int rt2 = 0; rt2 < kMfmaRows / 16; ++rt2) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = rt2 * 16 + grp * 4 + j;
      if (row < R) {
        const size_t pi = (((size_t)b * Hq + g * G + row / T) * T + row % T) * nparts + part;
        po[pi * kAttnD + dcol] = o[rt2][j];
      }
    }
  }
}

// One block of D threads per (token, q head): out = sum_c o_c e^(m_c - M) / sum_c l_c e^(m_c - M).
__global__ void attn_combine_kernel(const float* __restrict__ pm, const float* __restrict__ pl,
                                    const float* __restrict__ po, int T, int Hq, int nchunks,
                                    uint16_t* __restrict__ out) {
  const int m = blockIdx.x, h = blockIdx.y, d = threadIdx.x;
  const int b = m / T, i = m - b * T;
  const size_t base = (((size_t)b * Hq + h) * T + i) * nchunks;
  float mx = -INFINITY;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) mx = fmaxf(mx, pm[base + c]);
  float l = 0.0f, o = 0.0f;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) {
    const float mc = pm[base + c];
    const float w = mc == -INFINITY ? 0.0f : expf(mc - mx);
    l = l + pl[base + c] * w;
    o = o + po[(base + c) * kAttnD + d] * w;
  }
  out[((size_t)m * Hq + h) * kAttnD + d] = (uint16_t)f32_to_bf16_rne(o / l);
}

__global__ __launch_bounds__(kNormThreads) void silu_mul_kernel(const uint16_t* __restrict__ gu,
                                                                int I, uint16_t* __restrict__ out) {
  const int m = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= I) return;
  const float g = bf16_to_f32(gu[(size_t)m * 2 * I + j]);
  const float u = bf16_to_f32(gu[(size_t)m * 2 * I + I + j]);
  const float s = g / (1.0f + expf(-g));
  out[(size_t)m * I + j] = (uint16_t)f32_to_bf16_rne(s * u);
}

}  // namespace

int attn_chunks(int64_t pos0, int64_t T) { return (int)((pos0 + T + kAttnChunk - 1) / kAttnChunk); }

size_t attn_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t pos0) {
  const size_t rows = (size_t)B * Hq * T * attn_chunks(pos0, T);
  return align_up(rows * 4, kWsAlign) * 2 + align_up(rows * kAttnD * 4, kWsAlign);
}

bool attn_supported(int64_t Hq, int64_t Hkv, int64_t D, int64_t T) {
  return D == kAttnD && Hkv > 0 && Hq % Hkv == 0 && (Hq / Hkv) * T <= kAttnMaxRows;
}

hipError_t launch_embed(const int32_t* tok, const uint16_t* table, int64_t M, int64_t V, int64_t H,
                        float* h, hipStream_t st) {
  embed_kernel<<<dim3((unsigned)M), dim3(kNormThreads), 0, st>>>(tok, table, (int)V, (int)H, h);
  return hipGetLastError();
}

hipError_t launch_rmsnorm(float* h, const uint16_t* delta, const float* gamma, int64_t M, int64_t H,
                          float eps, uint16_t* out, hipStream_t st) {
  rmsnorm_kernel<<<dim3((unsigned)M), dim3(kNormThreads), 0, st>>>(h, delta, gamma, (int)H, eps, out);
  return hipGetLastError();
}

hipError_t launch_qk_rope_cache(const uint16_t* qkv, const float* q_gamma, const float* k_gamma,
                                int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t D,
                                int64_t pos0, int64_t Lmax, double log2_base, float eps,
                                uint16_t* q_out, uint16_t* k_cache, uint16_t* v_cache,
                                hipStream_t st) {
  qk_rope_cache_kernel<<<dim3((unsigned)(B * T), (unsigned)(Hq + 2 * Hkv)), dim3((unsigned)D), 0,
                         st>>>(qkv, q_gamma, k_gamma, (int)T, (int)Hq, (int)Hkv, (int)D, (int)pos0,
                               (int)Lmax, log2_base, eps, q_out, k_cache, v_cache);
  return hipGetLastError();
}


hipError_t launch_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t pos0, int64_t Lmax,
                            uint16_t* out, void* workspace, hipStream_t st) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attn_chunk_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      attn_lds_bytes(kAttnMaxRows));
  if (attr != hipSuccess) return attr;
  const int lds = attn_lds_bytes((int)((Hq / Hkv) * T));
  const int nch = attn_chunks(pos0, T);
  const size_t rows = (size_t)B * Hq * T * nch;
  char* ws = static_cast<char*>(workspace);
  float* pm = reinterpret_cast<float*>(ws);
  float* pl = reinterpret_cast<float*>(ws + align_up(rows * 4, kWsAlign));
  float* po = reinterpret_cast<float*>(ws + 2 * align_up(rows * 4, kWsAlign));
  int nparts = nch;
  if ((Hq / Hkv) * T <= kMfmaRows) {
    // chunks per workgroup: one while the chunk workgroups fit the device at
    // about four per compute unit, more (walked with a running softmax) when a
    // batch of sequences would need several rounds of them
    const int64_t chunk_wgs = (int64_t)nch * Hkv * B;
    const int cpw = (int)((chunk_wgs + kAttnResidentWgs - 1) / kAttnResidentWgs);
    nparts = (nch + cpw - 1) / cpw;
    attn_chunk_mfma_kernel<<<dim3((unsigned)nparts, (unsigned)Hkv, (unsigned)B), dim3(kAttnThreads),
                             0, st>>>(q, k_cache, v_cache, (int)T, (int)Hq, (int)Hkv, (int)pos0,
                                      (int)Lmax, nparts, cpw, 1.0f / sqrtf((float)kAttnD), pm, pl,
                                      po);
  } else {
    attn_chunk_kernel<<<dim3((unsigned)nch, (unsigned)Hkv, (unsigned)B), dim3(kAttnThreads), lds,
                        st>>>(q, k_cache, v_cache, (int)T, (int)Hq, (int)Hkv, (int)pos0, (int)Lmax,
                              nch, 1.0f / sqrtf((float)kAttnD), pm, pl, po);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_combine_kernel<<<dim3((unsigned)(B * T), (unsigned)Hq), dim3(kAttnD), 0, st>>>(
      pm, pl, po, (int)T, (int)Hq, nparts, out);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* gu, int64_t M, int64_t I, uint16_t* out, hipStream_t st) {
  silu_mul_kernel<<<dim3((unsigned)((I + kNormThreads - 1) / kNormThreads), (unsigned)M),
                    dim3(kNormThreads), 0, st>>>(gu, (int)I, out);
  return hipGetLastError();
}

}  // namespace quasar
