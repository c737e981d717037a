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
//   attn_wave_kernel     one KV head x a range of cached positions per
//                        wavefront: partial softmax (max, sum of exp,
//                        unnormalised output) of the group's query rows, both
//                        products on the matrix cores (groups of at most 32
//                        query rows)
//   attn_chunk_kernel    the same per 64 positions on the vector ALUs, for
//                        wider groups
//   attn_combine_kernel  merges the chunks of a query row
//   silu_mul_kernel      out = BF16(silu(gate) * up) over the gate_up output
#include <algorithm>

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

// The partials on the matrix cores, one wavefront per range of positions, for
// groups of at most 32 query rows (the Qwen3-8B window: 4 heads per KV head x 6
// positions = 24).  A wavefront walks `spw` steps of 32 keys with a running
// softmax per query row, and the four wavefronts of a workgroup (consecutive
// ranges) merge their maxima, sums and outputs in LDS at the end, so one
// partial per workgroup reaches memory; each step
//   scores  S^T = K Q^T, four tiles (2 key tiles x 2 query-row tiles) of
//           v_mfma_f32_16x16x32_bf16 over D = 128, operands straight from memory
//           (16 contiguous bytes of a key row and of a q row per lane).  Products
//           of BF16 values are exact in binary32.  Result register j of lane l is
//           key 4 (l / 16) + j of the tile, query row l % 16;
//   softmax per query row: the row's 32 scores sit in the four lanes l % 16 + 16 g
//           (8 each), so its maximum is a local max and two lane exchanges, and
//           every exponential is computed in the lane that holds the score;
//   P V     O^T += V^T P^T by v_mfma_f32_16x16x32_bf16.  The B operand of lane l is
//           query row l % 16 at the 8 keys this lane already holds (key slots
//           0..3 = keys 4 (l / 16) + j of the first key tile, 4..7 of the second),
//           so P never leaves the registers; the A operand is V^T at the same key
//           slots: two 8-byte LDS reads from this wavefront's transposed copy of
//           the values (dimension-major, keys contiguous), written there with
//           16-bit stores.  P (binary32, in [0, 1]) is split exactly into three BF16 parts
//           hi + mid + lo (truncations: 8 + 8 + 8 significant bits), each
//           multiplied in its own MFMA, so no product rounds P to BF16.
// The next step's keys and values are loaded before the current step's softmax.
// Result register j of the P V tiles is output dimension 4 (l / 16) + j of the
// tile for query row l % 16: the running output is rescaled per lane.
constexpr int kWaveKeys = 32;
// BF16 per row of the transposed values (one output dimension, 32 keys): rows
// 8 apart start 16 banks apart, so a store instruction (16 keys x 4 rows 8 apart)
// touches 32 distinct banks, and every row start is 8-byte aligned
constexpr int kWaveVtStride = 36;
constexpr int kAttnResidentWaves = 2048;  // two wavefronts per SIMD on 256 compute units
constexpr int kMfmaRows = 32;
constexpr int kAttnWaves = 4;                // wavefronts per workgroup, merged before the write
constexpr int kMergeStride = kAttnD + 4;     // floats per output row in the merge buffer
constexpr int kAttnWaveLds =
    std::max(kAttnWaves * kAttnD * kWaveVtStride * 2,
             (2 * kAttnWaves * kMfmaRows + (kAttnWaves - 1) * kMfmaRows * kMergeStride) * 4);

typedef __bf16 v8bf16 __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Steps of 32 keys per wavefront: one while the wavefronts of a launch are
// resident at once, more when a batch would need several rounds of them.
int attn_wave_steps(int64_t B, int64_t Hkv, int64_t klen) {
  const int64_t steps = (klen + kWaveKeys - 1) / kWaveKeys;
  const int64_t waves = steps * Hkv * B;
  return (int)std::max<int64_t>(1, (waves + kAttnResidentWaves - 1) / kAttnResidentWaves);
}

__device__ __forceinline__ uint32_t pack_hi16(float a, float b) {
  return (__float_as_uint(a) >> 16) | (__float_as_uint(b) & 0xffff0000u);
}

// Orders this wavefront's LDS stores before its later LDS loads (other lanes'
// data): LDS runs a wavefront's accesses in issue order, so only the compiler
// must keep them in place.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ __launch_bounds__(kAttnWaves * kWave, 2) void attn_wave_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_cache,
    const uint16_t* __restrict__ v_cache, int T, int Hq, int Hkv, int pos0, int Lmax, int spw,
    float scale, float* __restrict__ pm, float* __restrict__ pl, float* __restrict__ po) {
  // per wavefront: its transposed values; after the walk, reused for the merge
  __shared__ __align__(16) char lds[kAttnWaveLds];
  const int part = blockIdx.x, nparts = gridDim.x, g = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x % kWave, rl = lane & 15, grp = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  uint16_t* vt = reinterpret_cast<uint16_t*>(lds) + wave * kAttnD * kWaveVtStride;
  const int G = Hq / Hkv, R = G * T, klen = pos0 + T;
  const int t_begin = (part * kAttnWaves + wave) * spw * kWaveKeys;
  const int t_end = min(t_begin + spw * kWaveKeys, klen);  // t_end <= t_begin: no steps

  // B operands of the scores: query row rt * 16 + rl of the group at D values
  // 32 kk + 8 grp .. + 7; `vis` is the last key the row sees (-1: padding row)
  const buffer_rsrc qrs = make_rsrc(q + (size_t)b * T * Hq * kAttnD, (uint32_t)(T * Hq * kAttnD * 2));
  v4i qb[2][4];
  int vis[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = rt * 16 + rl;
    const int hh = r / T, i = r - hh * T;
    const int base = ((i * Hq + g * G + hh) * kAttnD + grp * 8) * 2;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) qb[rt][kk] = load16(qrs, r < R ? base + kk * 64 : kOutOfRange);
    vis[rt] = r < R ? pos0 + i : -1;
  }

  const size_t kv_head = ((size_t)b * Hkv + g) * Lmax * kAttnD;
  const int vkey = lane & 15, vcol8 = lane >> 4;
  v4i ka[2][4], vr[8];
  auto load_step = [&](int t0) {
    // keys t0 .. t0 + 31; those at or past klen read as zero (masked below)
    const uint32_t bytes = (uint32_t)min(kWaveKeys, klen - t0) * kAttnD * 2u;
    const buffer_rsrc krs = make_rsrc(k_cache + kv_head + (size_t)t0 * kAttnD, bytes);
    const buffer_rsrc vrs = make_rsrc(v_cache + kv_head + (size_t)t0 * kAttnD, bytes);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
        ka[kt][kk] = load16(krs, ((kt * 16 + rl) * kAttnD + kk * 32 + grp * 8) * 2);
    // value piece i of this lane: key vkey + 16 (i & 1), dimensions 8 vcol8 .. + 7
#pragma unroll
    for (int i = 0; i < 8; ++i)
      vr[i] = load16(vrs, ((vkey + 16 * (i & 1)) * kAttnD + (vcol8 + 4 * (i >> 1)) * 8) * 2);
  };
  if (t_begin < t_end) load_step(t_begin);

  float m_run[2] = {-INFINITY, -INFINITY}, l_part[2] = {0.0f, 0.0f};
  v4f o[8][2] = {};
  for (int t0 = t_begin; t0 < t_end; t0 += kWaveKeys) {
    v4f s[2][2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        s[rt][kt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          s[rt][kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf16, ka[kt][kk]), __builtin_bit_cast(v8bf16, qb[rt][kk]),
              s[rt][kt], 0, 0, 0);
      }
    wave_lds_sync();  // the previous step's reads of vt are done
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint16_t* dst = vt + (vcol8 + 4 * (i >> 1)) * 8 * kWaveVtStride + vkey + 16 * (i & 1);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const uint32_t w = (uint32_t)vr[i][c];
        dst[(2 * c) * kWaveVtStride] = (uint16_t)w;
        dst[(2 * c + 1) * kWaveVtStride] = (uint16_t)(w >> 16);
      }
    }
    if (t0 + kWaveKeys < t_end) load_step(t0 + kWaveKeys);

    // softmax pieces of query rows rt * 16 + rl; P split into BF16 parts
    v4i ph[2][3];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      float sv[8];
      float mx = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int key = t0 + kt * 16 + grp * 4 + j;
          sv[kt * 4 + j] = key <= vis[rt] ? s[rt][kt][j] * scale : -INFINITY;
          mx = fmaxf(mx, sv[kt * 4 + j]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16, kWave));
      mx = fmaxf(mx, __shfl_xor(mx, 32, kWave));
      const float m_new = fmaxf(m_run[rt], mx);
      const float fac = m_run[rt] == -INFINITY ? 0.0f : expf(m_run[rt] - m_new);
      float p[8], hi[8], mid[8], lo[8];
      float ls = 0.0f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = m_new == -INFINITY ? 0.0f : expf(sv[e] - m_new);
        ls = ls + p[e];
        hi[e] = __uint_as_float(__float_as_uint(p[e]) & 0xffff0000u);
        const float r1 = p[e] - hi[e];
        mid[e] = __uint_as_float(__float_as_uint(r1) & 0xffff0000u);
        lo[e] = r1 - mid[e];
      }
      l_part[rt] = l_part[rt] * fac + ls;
      m_run[rt] = m_new;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        ph[rt][0][d] = (int)pack_hi16(hi[2 * d], hi[2 * d + 1]);
        ph[rt][1][d] = (int)pack_hi16(mid[2 * d], mid[2 * d + 1]);
        ph[rt][2][d] = (int)pack_hi16(lo[2 * d], lo[2 * d + 1]);
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) o[dt][rt] = o[dt][rt] * fac;
    }
    wave_lds_sync();  // this step's values are in vt
    // A operands: V^T row dt * 16 + rl at key slots 0..7 of this lane's group
    // (keys 4 grp .. + 3 and 16 + 4 grp .. + 3)
    v4i va[8];
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const uint16_t* row = vt + (dt * 16 + rl) * kWaveVtStride + grp * 4;
      const int2 a = *reinterpret_cast<const int2*>(row);
      const int2 c = *reinterpret_cast<const int2*>(row + 16);
      va[dt] = v4i{a.x, a.y, c.x, c.y};
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int part3 = 0; part3 < 3; ++part3)
          o[dt][rt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(v8bf16, va[dt]), __builtin_bit_cast(v8bf16, ph[rt][part3]), o[dt][rt],
              0, 0, 0);
    }
  }

  // merge the workgroup's wavefronts: a common maximum per row, each
  // wavefront's sum and output rescaled to it; wavefronts 1.. hand theirs to
  // wavefront 0 through LDS, which adds them in wavefront order and writes
  float* mw = reinterpret_cast<float*>(lds);  // [waves][32] maxima
  float* lw = mw + kAttnWaves * kMfmaRows;    // [waves][32] rescaled sums
  float* ow = lw + kAttnWaves * kMfmaRows;    // [waves - 1][32][kMergeStride] outputs
  float l[2], mx[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    l[rt] = l_part[rt];
    l[rt] = l[rt] + __shfl_xor(l[rt], 16, kWave);
    l[rt] = l[rt] + __shfl_xor(l[rt], 32, kWave);
  }
  __syncthreads();  // every wavefront is done with its vt
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
    if (grp == 0) mw[wave * kMfmaRows + rt * 16 + rl] = m_run[rt];
  __syncthreads();
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = rt * 16 + rl;
    mx[rt] = mw[r];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) mx[rt] = fmaxf(mx[rt], mw[w * kMfmaRows + r]);
    const float f = m_run[rt] == -INFINITY ? 0.0f : expf(m_run[rt] - mx[rt]);
    if (grp == 0) lw[wave * kMfmaRows + r] = l[rt] * f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) o[dt][rt] = o[dt][rt] * f;
    if (wave > 0) {
      float* dst = ow + ((wave - 1) * kMfmaRows + r) * kMergeStride + grp * 4;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
        *reinterpret_cast<float4*>(dst + dt * 16) =
            make_float4(o[dt][rt][0], o[dt][rt][1], o[dt][rt][2], o[dt][rt][3]);
    }
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const int r = rt * 16 + rl;
    if (r >= R) continue;
    const size_t pi = (((size_t)b * Hq + g * G + r / T) * T + r % T) * nparts + part;
    if (grp == 0) {
      float ls = lw[r];
#pragma unroll
      for (int w = 1; w < kAttnWaves; ++w) ls = ls + lw[w * kMfmaRows + r];
      pm[pi] = mx[rt];
      pl[pi] = ls;
    }
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      float4 acc = make_float4(o[dt][rt][0], o[dt][rt][1], o[dt][rt][2], o[dt][rt][3]);
#pragma unroll
      for (int w = 1; w < kAttnWaves; ++w) {
        const float4 v = *reinterpret_cast<const float4*>(
            ow + ((w - 1) * kMfmaRows + r) * kMergeStride + grp * 4 + dt * 16);
        acc.x = acc.x + v.x;
        acc.y = acc.y + v.y;
        acc.z = acc.z + v.z;
        acc.w = acc.w + v.w;
      }
      *reinterpret_cast<float4*>(po + pi * kAttnD + grp * 4 + dt * 16) = acc;
    }
  }
}

// One block per (token, q head): out = sum_c o_c e^(m_c - M) / sum_c l_c e^(m_c - M)
// over the row's partials c, M their largest maximum.  G groups of 32 threads
// (G = blockDim.x / 32, 2 to 16: about four partials per group) take every G-th
// partial, 4 dimensions per thread with 16-byte loads, so that a row's loads are
// issued together; the groups' sums are then added in LDS in group order.
constexpr int kCombMaxThreads = 512;
constexpr int kCombMaxGroups = kCombMaxThreads / (kAttnD / 4);

int attn_combine_threads(int64_t nparts) {
  int g = 1;
  while (g < kCombMaxGroups && 4 * g < nparts) g *= 2;
  return std::max(g * (kAttnD / 4), kWave);
}

__global__ __launch_bounds__(kCombMaxThreads) void attn_combine_kernel(
    const float* __restrict__ pm, const float* __restrict__ pl, const float* __restrict__ po, int T,
    int Hq, int nparts, uint16_t* __restrict__ out) {
  __shared__ float red[kCombMaxThreads / kWave];
  __shared__ float4 osum[kCombMaxGroups][kAttnD / 4];
  __shared__ float lsum[kCombMaxGroups];
  const int m = blockIdx.x, h = blockIdx.y, tid = threadIdx.x;
  const int nthreads = blockDim.x, ngroups = nthreads / (kAttnD / 4), nwaves = nthreads / kWave;
  const int b = m / T, i = m - b * T;
  const size_t base = (((size_t)b * Hq + h) * T + i) * nparts;
  float mx = -INFINITY;
  for (int c = tid; c < nparts; c += nthreads) mx = fmaxf(mx, pm[base + c]);
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off, kWave));
  if (tid % kWave == 0) red[tid / kWave] = mx;
  __syncthreads();
  mx = red[0];
  for (int w = 1; w < nwaves; ++w) mx = fmaxf(mx, red[w]);
  const int grp = tid / (kAttnD / 4), d4 = tid % (kAttnD / 4);
  float l = 0.0f;
  float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
#pragma unroll 4
  for (int c = grp; c < nparts; c += ngroups) {
    const float mc = pm[base + c];
    const float w = mc == -INFINITY ? 0.0f : expf(mc - mx);
    l = l + pl[base + c] * w;
    const float4 v = *reinterpret_cast<const float4*>(po + (base + c) * kAttnD + d4 * 4);
    o.x = o.x + v.x * w;
    o.y = o.y + v.y * w;
    o.z = o.z + v.z * w;
    o.w = o.w + v.w * w;
  }
  osum[grp][d4] = o;
  if (d4 == 0) lsum[grp] = l;
  __syncthreads();
  const float* os = reinterpret_cast<const float*>(&osum[0][0]);
  for (int d = tid; d < kAttnD; d += nthreads) {
    float acc = 0.0f, L = 0.0f;
    for (int g2 = 0; g2 < ngroups; ++g2) {
      acc = acc + os[g2 * kAttnD + d];
      L = L + lsum[g2];
    }
    out[((size_t)m * Hq + h) * kAttnD + d] = (uint16_t)f32_to_bf16_rne(acc / L);
  }
}

// kGated: the columns of gu are in the gated order (16-column tiles of 8 gate
// then 8 up columns) instead of [gate | up].
template <bool kGated>
__global__ __launch_bounds__(kNormThreads) void silu_mul_kernel(const uint16_t* __restrict__ gu,
                                                                int I, uint16_t* __restrict__ out) {
  const int m = blockIdx.y;
  const int j = blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= I) return;
  const int gc = kGated ? (j >> 3) * 16 + (j & 7) : j;
  const int uc = kGated ? gc + 8 : I + j;
  const float g = bf16_to_f32(gu[(size_t)m * 2 * I + gc]);
  const float u = bf16_to_f32(gu[(size_t)m * 2 * I + uc]);
  const float s = g / (1.0f + expf(-g));
  out[(size_t)m * I + j] = (uint16_t)f32_to_bf16_rne(s * u);
}

}  // namespace

int attn_chunks(int64_t pos0, int64_t T) { return (int)((pos0 + T + kAttnChunk - 1) / kAttnChunk); }

// Partials per query row: position ranges of the wavefront kernel, or 64-position
// chunks of the vector-ALU kernel.
static int64_t attn_parts(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t pos0) {
  const int64_t klen = pos0 + T;
  if ((Hq / Hkv) * T > kMfmaRows) return attn_chunks(pos0, T);
  const int64_t steps = (klen + kWaveKeys - 1) / kWaveKeys;
  const int64_t spw = attn_wave_steps(B, Hkv, klen);
  const int64_t wave_parts = (steps + spw - 1) / spw;
  return (wave_parts + kAttnWaves - 1) / kAttnWaves;
}

size_t attn_workspace_bytes(int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t pos0) {
  const size_t rows = (size_t)B * Hq * T * attn_parts(B, T, Hq, Hkv, pos0);
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
  const int64_t nparts = attn_parts(B, T, Hq, Hkv, pos0);
  const size_t rows = (size_t)B * Hq * T * nparts;
  char* ws = static_cast<char*>(workspace);
  float* pm = reinterpret_cast<float*>(ws);
  float* pl = reinterpret_cast<float*>(ws + align_up(rows * 4, kWsAlign));
  float* po = reinterpret_cast<float*>(ws + 2 * align_up(rows * 4, kWsAlign));
  const float scale = 1.0f / sqrtf((float)kAttnD);
  if ((Hq / Hkv) * T <= kMfmaRows) {
    const int spw = attn_wave_steps(B, Hkv, pos0 + T);
    attn_wave_kernel<<<dim3((unsigned)nparts, (unsigned)Hkv, (unsigned)B), dim3(kAttnWaves * kWave),
                       0, st>>>(q, k_cache, v_cache, (int)T, (int)Hq, (int)Hkv, (int)pos0,
                                (int)Lmax, spw, scale, pm, pl, po);
  } else {
    attn_chunk_kernel<<<dim3((unsigned)nparts, (unsigned)Hkv, (unsigned)B), dim3(kAttnThreads), lds,
                        st>>>(q, k_cache, v_cache, (int)T, (int)Hq, (int)Hkv, (int)pos0, (int)Lmax,
                              (int)nparts, scale, pm, pl, po);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_combine_kernel<<<dim3((unsigned)(B * T), (unsigned)Hq),
                        dim3((unsigned)attn_combine_threads(nparts)), 0, st>>>(
      pm, pl, po, (int)T, (int)Hq, (int)nparts, out);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* gu, int64_t M, int64_t I, uint16_t* out, hipStream_t st) {
  silu_mul_kernel<false><<<dim3((unsigned)((I + kNormThreads - 1) / kNormThreads), (unsigned)M),
                           dim3(kNormThreads), 0, st>>>(gu, (int)I, out);
  return hipGetLastError();
}

hipError_t launch_silu_mul_gated(const uint16_t* gu, int64_t M, int64_t I, uint16_t* out,
                                 hipStream_t st) {
  silu_mul_kernel<true><<<dim3((unsigned)((I + kNormThreads - 1) / kNormThreads), (unsigned)M),
                          dim3(kNormThreads), 0, st>>>(gu, (int)I, out);
  return hipGetLastError();
}

}  // namespace quasar
