// Verification decision over the dequantized BF16 logits of the 1+k verify
// positions: greedy at T = 0 [Quasar, ko page §4, "Qwen3 (Greedy, T=0)"] or
// rejection sampling that keeps the verifier's distribution [pt page §2 item 4;
// zh page §2 "lossless rejection sampling"].
//
// Pass 1 (grid chunks x rows): every workgroup scans one chunk of one logits
// row and writes the chunk's (max, lowest argmax) and, for T > 0, the chunk's
// sum of exp((l - max_chunk) / T).
// Pass 2 (grid B): one workgroup per sequence merges the chunk partials of its
// k+1 rows, takes the accept decisions in draft order and picks the next token
// (argmax, or an inverse-CDF draw over the residual in index order).
//
// Pass 2 also serves the LM head whose own epilogue produced the partials
// (one chunk per workgroup of that kernel): chunk c then starts at logit
// 16 (c q + floor(c r / G)) instead of 2048 c.  Chunks are at most 2048 wide
// either way.
#include <float.h>
#include <limits.h>

#include "quasar_device.hpp"
#include "quasar_internal.hpp"

namespace quasar {
namespace {

constexpr int kThreads = 256;
constexpr int kChunk = kAcceptChunk;  // logits per pass-1 workgroup (8 per thread)
constexpr int kMaxRows = 64;  // k + 1 <= 64

struct ArgMax {
  float v;
  int idx;
};

// larger value wins; equal values (as reals, so -0 == +0) go to the lower index
__device__ __forceinline__ ArgMax better(ArgMax a, ArgMax b) {
  if (b.v > a.v || (b.v == a.v && b.idx < a.idx)) return b;
  return a;
}

__device__ __forceinline__ ArgMax wave_argmax(ArgMax a) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    ArgMax o;
    o.v = __shfl_xor(a.v, off, kWave);
    o.idx = __shfl_xor(a.idx, off, kWave);
    a = better(a, o);
  }
  return a;
}

__device__ ArgMax block_argmax(ArgMax a, float* sv, int* si) {
  a = wave_argmax(a);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (lane == 0) {
    sv[wave] = a.v;
    si[wave] = a.idx;
  }
  __syncthreads();
  ArgMax r{sv[0], si[0]};
  for (int w = 1; w < kThreads / kWave; ++w) r = better(r, ArgMax{sv[w], si[w]});
  __syncthreads();
  return r;
}

__device__ float block_sum(float v, float* sv) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (lane == 0) sv[wave] = v;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < kThreads / kWave; ++w) r += sv[w];
  __syncthreads();
  return r;
}

template <bool kSample>
__global__ __launch_bounds__(kThreads) void accept_partial_kernel(
    const uint16_t* __restrict__ logits, int64_t V, int chunks, float inv_t,
    float* __restrict__ pmax, int32_t* __restrict__ pidx, float* __restrict__ psum) {
  __shared__ float sv[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  const int c = blockIdx.x;
  const int64_t row = blockIdx.y;
  const uint16_t* lr = logits + row * V;
  const int64_t j0 = (int64_t)c * kChunk;
  const int64_t j1 = min(V, j0 + kChunk);
  ArgMax best{-FLT_MAX, INT_MAX};
  float vals[kChunk / kThreads];
#pragma unroll
  for (int e = 0; e < kChunk / kThreads; ++e) {
    const int64_t j = j0 + (int64_t)e * kThreads + threadIdx.x;
    vals[e] = -FLT_MAX;
    if (j < j1) {
      vals[e] = bf16_to_f32(lr[j]);
      best = better(best, ArgMax{vals[e], (int)j});
    }
  }
  best = block_argmax(best, sv, si);
  const int64_t slot = row * chunks + c;
  if (kSample) {
    float sum = 0.0f;
#pragma unroll
    for (int e = 0; e < kChunk / kThreads; ++e) {
      const int64_t j = j0 + (int64_t)e * kThreads + threadIdx.x;
      if (j < j1) sum += expf((vals[e] - best.v) * inv_t);
    }
    sum = block_sum(sum, sv);
    if (threadIdx.x == 0) psum[slot] = sum;
  }
  if (threadIdx.x == 0) {
    pmax[slot] = best.v;
    pidx[slot] = best.idx;
  }
}

// Chunk c covers logits [start(c), start(c + 1)) of a row: start(c) =
// unit (c q + floor(c r / G)), capped at V.
struct ChunkGeometry {
  int unit, q, r, G;
};

__device__ __forceinline__ int64_t chunk_start(const ChunkGeometry& cg, int c, int64_t V) {
  const int64_t u = (int64_t)c * cg.q + (int64_t)c * cg.r / cg.G;
  return min(V, u * cg.unit);
}

// the chunk holding logit j (0 <= j < V): the last c with start(c) <= j
__device__ __forceinline__ int chunk_of(const ChunkGeometry& cg, int chunks, int64_t j, int64_t V) {
  int lo = 0, hi = chunks - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (chunk_start(cg, mid, V) <= j) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Inclusive prefix sum over the workgroup (thread order); `wsum` holds one
// float per wavefront.  Ends with a barrier, so `wsum` can be reused.
__device__ float block_incl_scan(float v, float* wsum) {
  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const float o = __shfl_up(v, off, kWave);
    if (lane >= off) v += o;
  }
  if (lane == kWave - 1) wsum[wave] = v;
  __syncthreads();
  float add = 0.0f;
  for (int w = 0; w < wave; ++w) add += wsum[w];
  __syncthreads();
  return v + add;
}

template <bool kSample>
__global__ __launch_bounds__(kThreads) void accept_finalize_kernel(
    const uint16_t* __restrict__ logits, const int32_t* __restrict__ draft, int k, int64_t V,
    int chunks, ChunkGeometry cg, float inv_t, const float* __restrict__ uniforms,
    const float* __restrict__ pmax, const int32_t* __restrict__ pidx,
    const float* __restrict__ psum, int32_t* __restrict__ accept_len,
    int32_t* __restrict__ next_token, int32_t* __restrict__ argmax_out,
    float* __restrict__ p_draft_out) {
  __shared__ float sv[kThreads / kWave];
  __shared__ int si[kThreads / kWave];
  __shared__ int s_g[kMaxRows], s_d[kMaxRows];
  __shared__ float s_m[kMaxRows], s_z[kMaxRows], s_p[kMaxRows], s_u[kMaxRows];
  __shared__ int s_L, s_cstar, s_found, s_fallback;
  __shared__ float s_before, s_target;
  __shared__ float s_run[kThreads];

  const int b = blockIdx.x, tid = threadIdx.x;
  const int kp1 = k + 1;
  // the sequence's drafts and uniforms, loaded in parallel
  if (tid < k) s_d[tid] = draft[(int64_t)b * k + tid];
  if (kSample && tid < kp1) s_u[tid] = uniforms[(int64_t)b * kp1 + tid];

  // ---- merge the chunk partials of every verify position
  if (kp1 <= 8 && chunks <= kThreads) {
    // thread c holds chunk c of every row: all loads are issued before any
    // reduction, so their latency is paid once rather than once per row
    float vm[8], vs[8];
    int vi[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      vm[i] = -FLT_MAX;
      vi[i] = INT_MAX;
      vs[i] = 0.0f;
      if (i < kp1 && tid < chunks) {
        const int64_t slot = ((int64_t)b * kp1 + i) * chunks + tid;
        vm[i] = pmax[slot];
        vi[i] = pidx[slot];
        if (kSample) vs[i] = psum[slot];
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      if (i < kp1) {
        const ArgMax a = block_argmax(ArgMax{vm[i], vi[i]}, sv, si);
        float z = 0.0f;
        if (kSample) z = block_sum(tid < chunks ? vs[i] * expf((vm[i] - a.v) * inv_t) : 0.0f, sv);
        if (tid == 0) {
          s_g[i] = a.idx;
          s_m[i] = a.v;
          s_z[i] = z;
        }
      }
    }
  } else {
    for (int i = 0; i < kp1; ++i) {
      const int64_t row = (int64_t)b * kp1 + i;
      ArgMax a{-FLT_MAX, INT_MAX};
      for (int c = tid; c < chunks; c += kThreads)
        a = better(a, ArgMax{pmax[row * chunks + c], pidx[row * chunks + c]});
      a = block_argmax(a, sv, si);
      float z = 0.0f;
      if (kSample) {
        float part = 0.0f;
        for (int c = tid; c < chunks; c += kThreads)
          part += psum[row * chunks + c] * expf((pmax[row * chunks + c] - a.v) * inv_t);
        z = block_sum(part, sv);
      }
      if (tid == 0) {
        s_g[i] = a.idx;
        s_m[i] = a.v;
        s_z[i] = z;
      }
    }
  }
  __syncthreads();

  if (!kSample) {
    if (tid == 0) {
      int L = 0;
      while (L < k && s_d[L] == s_g[L]) ++L;
      accept_len[b] = L;
      next_token[b] = s_g[L];
    }
    if (argmax_out)
      for (int i = tid; i < kp1; i += kThreads) argmax_out[(int64_t)b * kp1 + i] = s_g[i];
    return;
  }

  // ---- rejection: p_i(draft i) for every draft in parallel, then the
  // accept decisions in draft order
  if (tid < k) {
    const int d = s_d[tid];
    float p = 0.0f;
    if (d >= 0 && d < V) {
      const float l = bf16_to_f32(logits[((int64_t)b * kp1 + tid) * V + d]);
      p = expf((l - s_m[tid]) * inv_t) / s_z[tid];
    }
    s_p[tid] = p;
    if (p_draft_out) p_draft_out[(int64_t)b * k + tid] = p;
  }
  __syncthreads();
  if (tid == 0) {
    int L = k;
    for (int i = 0; i < k; ++i)
      if (!(s_u[i] < s_p[i])) {
        L = i;
        break;
      }
    s_L = L;
  }
  __syncthreads();
  const int L = s_L;
  const int64_t row = (int64_t)b * kp1 + L;
  const float m = s_m[L];
  int d_ex = -1;  // token removed from the residual (the rejected draft)
  if (L < k) {
    const int d = s_d[L];
    if (d >= 0 && d < V) d_ex = d;
  }
  const int c_ex = d_ex >= 0 ? chunk_of(cg, chunks, d_ex, V) : -1;
  // the chunk holding the rejected draft: its sum without that token
  float ex_sum = 0.0f;
  if (c_ex >= 0) {
    float part = 0.0f;
    const int64_t j1 = chunk_start(cg, c_ex + 1, V);
    for (int64_t j = chunk_start(cg, c_ex, V) + tid; j < j1; j += kThreads)
      if (j != d_ex) part += expf((bf16_to_f32(logits[row * V + j]) - m) * inv_t);
    ex_sum = block_sum(part, sv);
  }
  // ---- the chunk holding the draw: the first whose running sum of chunk sums
  // (rescaled to the row max) passes u * total
  if (tid == 0) {
    s_found = INT_MAX;
    s_fallback = -1;
  }
  if (chunks <= kThreads) {
    float sc = 0.0f;
    if (tid < chunks)
      sc = (tid == c_ex) ? ex_sum
                         : psum[row * chunks + tid] * expf((pmax[row * chunks + tid] - m) * inv_t);
    const float incl = block_incl_scan(sc, sv);  // ends with a barrier
    s_run[tid] = incl;
    __syncthreads();
    const float total = s_run[chunks - 1];
    const float target = s_u[k] * total;
    if (tid < chunks) {
      if (incl > target) atomicMin(&s_found, tid);
      if (sc > 0.0f) atomicMax(&s_fallback, tid);
    }
    __syncthreads();
    if (tid == 0) {
      int cstar = s_found;
      float before;
      if (cstar != INT_MAX) {
        before = cstar > 0 ? s_run[cstar - 1] : 0.0f;
      } else {  // rounding pushed the target past the last chunk
        cstar = s_fallback >= 0 ? s_fallback : 0;
        before = total;
      }
      s_cstar = cstar;
      s_before = before;
      s_target = target;
      s_found = INT_MAX;
      s_fallback = -1;
    }
  } else if (tid == 0) {
    float total = 0.0f;
    for (int c = 0; c < chunks; ++c)
      total += (c == c_ex) ? ex_sum : psum[row * chunks + c] * expf((pmax[row * chunks + c] - m) * inv_t);
    const float target = s_u[k] * total;
    float cum = 0.0f;
    int cstar = -1, last_nz = 0;
    float before = 0.0f;
    for (int c = 0; c < chunks; ++c) {
      const float sc = (c == c_ex) ? ex_sum : psum[row * chunks + c] * expf((pmax[row * chunks + c] - m) * inv_t);
      if (sc > 0.0f) last_nz = c;
      if (cstar < 0 && cum + sc > target) {
        cstar = c;
        before = cum;
      }
      cum += sc;
    }
    if (cstar < 0) {  // rounding pushed the target past the last chunk
      cstar = last_nz;
      before = cum;
    }
    s_cstar = cstar;
    s_before = before;
    s_target = target;
    s_found = INT_MAX;
    s_fallback = -1;
  }
  __syncthreads();
  // ---- scan the chosen chunk in index order: thread t owns 8 consecutive logits
  const int64_t base = chunk_start(cg, s_cstar, V);
  const int64_t end = chunk_start(cg, s_cstar + 1, V);  // at most kChunk past base
  constexpr int E = kChunk / kThreads;
  float rr[E];
  float run = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int64_t j = base + (int64_t)tid * E + e;
    rr[e] = 0.0f;
    if (j < end && j != d_ex) rr[e] = expf((bf16_to_f32(logits[row * V + j]) - m) * inv_t);
    run += rr[e];
  }
  const float excl = block_incl_scan(run, sv) - run;  // this thread's exclusive prefix
  float cum = s_before + excl;
  const float target = s_target;
  int found = INT_MAX, nz = -1;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = (int)(base + tid * E + e);
    cum += rr[e];
    if (rr[e] > 0.0f) {
      nz = j;
      if (found == INT_MAX && cum > target) found = j;
    }
  }
  if (found != INT_MAX) atomicMin(&s_found, found);
  if (nz >= 0) atomicMax(&s_fallback, nz);
  __syncthreads();
  if (tid == 0) {
    accept_len[b] = L;
    next_token[b] = s_found != INT_MAX ? s_found : (s_fallback >= 0 ? s_fallback : 0);
  }
}

}  // namespace

AcceptPlan plan_accept(int64_t B, int64_t k, int64_t V) {
  AcceptPlan p{};
  p.B = B;
  p.k = k;
  p.V = V;
  p.rows = B * (k + 1);
  p.chunk_len = kChunk;
  p.chunks = (int)((V + kChunk - 1) / kChunk);
  p.unit = kChunk;
  p.cq = 1;
  p.cr = 0;
  p.cG = 1;
  const size_t slots = (size_t)p.rows * p.chunks;
  size_t off = 0;
  p.off_max = off;
  off = align_up(off + slots * sizeof(float), kWsAlign);
  p.off_idx = off;
  off = align_up(off + slots * sizeof(int32_t), kWsAlign);
  p.off_sum = off;
  off = align_up(off + slots * sizeof(float), kWsAlign);
  p.bytes = B == 0 ? 0 : off;
  return p;
}

hipError_t launch_accept(const AcceptPlan& p, const uint16_t* logits, const int32_t* draft,
                         float temperature, const float* uniforms, int32_t* accept_len,
                         int32_t* next_token, int32_t* argmax_out, float* p_draft_out,
                         void* workspace, hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  float* pmax = reinterpret_cast<float*>(ws + p.off_max);
  int32_t* pidx = reinterpret_cast<int32_t*>(ws + p.off_idx);
  float* psum = reinterpret_cast<float*>(ws + p.off_sum);
  const bool sample = temperature > 0.0f;
  const float inv_t = sample ? 1.0f / temperature : 0.0f;
  const dim3 g1((unsigned)p.chunks, (unsigned)p.rows), blk(kThreads);
  if (sample)
    accept_partial_kernel<true><<<g1, blk, 0, st>>>(logits, p.V, p.chunks, inv_t, pmax, pidx, psum);
  else
    accept_partial_kernel<false><<<g1, blk, 0, st>>>(logits, p.V, p.chunks, inv_t, pmax, pidx, psum);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_accept_finalize(p, logits, draft, temperature, uniforms, accept_len, next_token,
                                argmax_out, p_draft_out, pmax, pidx, psum, st);
}

hipError_t launch_accept_finalize(const AcceptPlan& p, const uint16_t* logits,
                                  const int32_t* draft, float temperature, const float* uniforms,
                                  int32_t* accept_len, int32_t* next_token, int32_t* argmax_out,
                                  float* p_draft_out, const float* pmax, const int32_t* pidx,
                                  const float* psum, hipStream_t st) {
  const bool sample = temperature > 0.0f;
  const float inv_t = sample ? 1.0f / temperature : 0.0f;
  const ChunkGeometry cg{p.unit, p.cq, p.cr, p.cG};
  const dim3 g2((unsigned)p.B), blk(kThreads);
  if (sample)
    accept_finalize_kernel<true><<<g2, blk, 0, st>>>(logits, draft, (int)p.k, p.V, p.chunks, cg,
                                                     inv_t, uniforms, pmax, pidx, psum, accept_len,
                                                     next_token, argmax_out, p_draft_out);
  else
    accept_finalize_kernel<false><<<g2, blk, 0, st>>>(logits, draft, (int)p.k, p.V, p.chunks, cg,
                                                      inv_t, uniforms, pmax, pidx, psum,
                                                      accept_len, next_token, argmax_out,
                                                      p_draft_out);
  return hipGetLastError();
}

}  // namespace quasar
