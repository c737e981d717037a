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
//   attn_chunk_kernel    one KV head x 64 cached positions: partial softmax
//                        (max, sum of exp, unnormalised output) of the group's
//                        query rows
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

// One block per row.  mean(h^2) is a binary32 sum of squares in a fixed
// order per thread, then across the block.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(float* __restrict__ h,
                                                               const uint16_t* __restrict__ delta,
                                                               const float* __restrict__ gamma,
                                                               int H, float eps,
                                                               uint16_t* __restrict__ out) {
  __shared__ float red[kNormThreads / kWave];
  const int m = blockIdx.x;
  float* hr = h + (size_t)m * H;
  float ss = 0.0f;
  for (int j = threadIdx.x; j < H; j += blockDim.x) {
    float v = hr[j];
    if (delta) {
      v = v + bf16_to_f32(delta[(size_t)m * H + j]);
      hr[j] = v;
    }
    ss = ss + v * v;
  }
  const float tot = block_sum(ss, red);
  const float r = 1.0f / sqrtf(tot / (float)H + eps);
  for (int j = threadIdx.x; j < H; j += blockDim.x)
    out[(size_t)m * H + j] = (uint16_t)f32_to_bf16_rne(hr[j] * r * gamma[j]);
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
constexpr int kAttnChunk = 64;
constexpr int kAttnThreads = 256;
constexpr int kAttnMaxRows = 64;  // (Hq / Hkv) * T
constexpr int kAttnD = 128;

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
  float* qs = reinterpret_cast<float*>(smem);          // [R][D]
  float* ks = qs + kAttnMaxRows * kAttnD;              // [64][D + 1]
  float* vs = ks + kAttnChunk * (kAttnD + 1);          // [64][D]
  float* ps = vs + kAttnChunk * kAttnD;                // [R][64]
  const int tid = threadIdx.x;
  for (int e = tid; e < R * kAttnD; e += kAttnThreads) {
    const int r = e / kAttnD, d = e - r * kAttnD;
    const int hh = r / T, i = r - hh * T;
    const int m = b * T + i, h = g * G + hh;
    qs[e] = bf16_to_f32(q[((size_t)m * Hq + h) * kAttnD + d]);
  }
  const size_t kv0 = (((size_t)b * Hkv + g) * Lmax + t0) * kAttnD;
  for (int e = tid; e < nt * kAttnD; e += kAttnThreads) {
    const int t = e / kAttnD, d = e - t * kAttnD;
    ks[t * (kAttnD + 1) + d] = bf16_to_f32(k_cache[kv0 + e]);
    vs[e] = bf16_to_f32(v_cache[kv0 + e]);
  }
  __syncthreads();
  // scores: thread pairs (row, key)
  for (int e = tid; e < R * kAttnChunk; e += kAttnThreads) {
    const int r = e / kAttnChunk, t = e - r * kAttnChunk;
    const int i = r % T;
    float sc = -INFINITY;
    if (t < nt && t0 + t <= pos0 + i) {
      float acc = 0.0f;
      const float* qr = qs + r * kAttnD;
      const float* kr = ks + t * (kAttnD + 1);
      for (int d = 0; d < kAttnD; ++d) acc = acc + qr[d] * kr[d];
      sc = acc * scale;
    }
    ps[e] = sc;
  }
  __syncthreads();
  // per row: max, exp, sum (one wavefront per row, rows round-robin)
  const int wave = tid / kWave, lane = tid % kWave;
  for (int r = wave; r < R; r += kAttnThreads / kWave) {
    float* pr = ps + r * kAttnChunk;
    float mx = -INFINITY;
    for (int t = lane; t < kAttnChunk; t += kWave) mx = fmaxf(mx, pr[t]);
    mx = wave_max(mx);
    float sum = 0.0f;
    for (int t = lane; t < kAttnChunk; t += kWave) {
      const float p = mx == -INFINITY ? 0.0f : expf(pr[t] - mx);
      pr[t] = p;
      sum = sum + p;
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
    if (lane == 0) {
      const size_t pi = (((size_t)b * Hq + g * G + r / T) * T + r % T) * nchunks + c;
      pm[pi] = mx;
      pl[pi] = sum;
    }
  }
  __syncthreads();
  // unnormalised outputs: thread pairs (row, d), keys in order
  for (int e = tid; e < R * kAttnD; e += kAttnThreads) {
    const int r = e / kAttnD, d = e - r * kAttnD;
    const float* pr = ps + r * kAttnChunk;
    float acc = 0.0f;
    for (int t = 0; t < nt; ++t) acc = acc + pr[t] * vs[t * kAttnD + d];
    const size_t pi = (((size_t)b * Hq + g * G + r / T) * T + r % T) * nchunks + c;
    po[pi * kAttnD + d] = acc;
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
  for (int c = 0; c < nchunks; ++c) mx = fmaxf(mx, pm[base + c]);
  float l = 0.0f, o = 0.0f;
  for (int c = 0; c < nchunks; ++c) {
    const float mc = pm[base + c];
    if (mc == -INFINITY) continue;
    const float w = expf(mc - mx);
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

constexpr int kAttnLds =
    (kAttnMaxRows * kAttnD + kAttnChunk * (kAttnD + 1) + kAttnChunk * kAttnD +
     kAttnMaxRows * kAttnChunk) * 4;

hipError_t launch_attention(const uint16_t* q, const uint16_t* k_cache, const uint16_t* v_cache,
                            int64_t B, int64_t T, int64_t Hq, int64_t Hkv, int64_t pos0, int64_t Lmax,
                            uint16_t* out, void* workspace, hipStream_t st) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&attn_chunk_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
      kAttnLds);
  if (attr != hipSuccess) return attr;
  const int nch = attn_chunks(pos0, T);
  const size_t rows = (size_t)B * Hq * T * nch;
  char* ws = static_cast<char*>(workspace);
  float* pm = reinterpret_cast<float*>(ws);
  float* pl = reinterpret_cast<float*>(ws + align_up(rows * 4, kWsAlign));
  float* po = reinterpret_cast<float*>(ws + 2 * align_up(rows * 4, kWsAlign));
  attn_chunk_kernel<<<dim3((unsigned)nch, (unsigned)Hkv, (unsigned)B), dim3(kAttnThreads), kAttnLds,
                      st>>>(q, k_cache, v_cache, (int)T, (int)Hq, (int)Hkv, (int)pos0, (int)Lmax, nch,
                            1.0f / sqrtf((float)kAttnD), pm, pl, po);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  attn_combine_kernel<<<dim3((unsigned)(B * T), (unsigned)Hq), dim3(kAttnD), 0, st>>>(
      pm, pl, po, (int)T, (int)Hq, nch, out);
  return hipGetLastError();
}

hipError_t launch_silu_mul(const uint16_t* gu, int64_t M, int64_t I, uint16_t* out, hipStream_t st) {
  silu_mul_kernel<<<dim3((unsigned)((I + kNormThreads - 1) / kNormThreads), (unsigned)M),
                    dim3(kNormThreads), 0, st>>>(gu, (int)I, out);
  return hipGetLastError();
}

}  // namespace quasar
