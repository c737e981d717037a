// One-launch W8A8 SmoothQuant linear for the verify window (M <= 8 tokens):
// online smoothing + dynamic per-token INT8 quantization of the BF16
// activations, INT8 x INT8 -> INT32 MFMA product against the resident INT8
// weights, and BF16 dequantization, in a single kernel
// [Quasar, pt page §2 execution pipeline items 2-4; zh page §2 items 2-3].
//
// Why one launch: a verify step runs ~145 of these linears back to back and a
// kernel boundary costs ~1.6 us on MI355X even inside a HIP graph, so the
// activation quantizer runs as the prologue of every workgroup instead of as a
// kernel of its own.  It reads only the M x K activations (tens of KB, L2
// resident) while the INT8 weight stream -- the only large traffic -- is
// already in flight.
//
// Work decomposition (persistent grid, one workgroup per compute unit):
//   * a tile is 16 output channels x all of K; workgroup b handles tiles
//     b, b + G, b + 2G, ... (G = grid size);
//   * wavefronts are specialized.  A compute unit keeps only ~32-64 KB of
//     vector-memory misses in flight, and a wavefront that issues beyond that
//     stalls at issue until data returns.  So four *streamer* wavefronts own
//     the weight stream: streamer w owns chunks [w*8*NPH, (w+1)*8*NPH) of 64 K
//     positions, in NPH phases of 8 chunks, double-buffered (the next phase is
//     in flight while the current one is multiplied).  Each chunk is one
//     contiguous 1 KB of the tile-packed weights (one 128-bit load per lane,
//     already in MFMA A-operand order), loaded with the streaming (nt) policy.
//     Stalling at issue costs a streamer nothing;
//   * NH *helper* wavefronts quantize the activations and finish the tiles.
//     They load the activations first (a barrier orders these loads before
//     any weight load of the compute unit: loads return in issue order), form
//     xs = RN32(x * s), reduce the per-token absmax (DPP within a wavefront,
//     then an LDS counter among the helpers -- not a workgroup barrier, which
//     would wait for the stalled streamers) and write the INT8 codes into an
//     LDS matrix that feeds the MFMA B operand.  Helpers issue no load behind
//     the weight stream;
//   * per tile the streamers' 16x16 INT32 partials (and the tile's weight
//     scales, fetched by streamer 0 with its last phase) go to LDS, and 64
//     helper threads apply the dequant epilogue, 4 channels (8 bytes) per
//     store.
#include "quasar_device.hpp"
#include "quasar_internal.hpp"

namespace quasar {
namespace {

constexpr int kMaxMT = 8;      // token rows the one-launch kernel handles
constexpr int kPH = 8;         // chunks per weight phase (8 KB per wavefront)
constexpr int kStreamers = 4;  // weight-streaming wavefronts per workgroup
constexpr int kMaxHelpers = 8;

// Variants by K (NPH phases per streamer and tile, NBUF phase buffers per
// streamer, NH helper wavefronts, UP activation pieces of 8 K positions per
// helper thread and token row):
//   K <= 4096:  NPH 2, NBUF 2, NH 4, UP 2  (64 KB of weights requested per CU)
//   K <= 8192:  NPH 4, NBUF 2, NH 8, UP 2  (64 KB)
//   K <= 12288: NPH 6, NBUF 3, NH 8, UP 3  (96 KB)
// before the code matrix exists: larger K means a longer quantization prologue,
// during which the buffers keep the compute unit's share of HBM busy.
__host__ __device__ constexpr int variant_nh(int nph) { return nph == 2 ? 4 : 8; }
__host__ __device__ constexpr int variant_up(int nph) { return nph == 6 ? 3 : 2; }
__host__ __device__ constexpr int variant_nbuf(int nph) { return nph == 6 ? 3 : 2; }
__host__ __device__ constexpr int variant_kmax(int nph) { return kStreamers * kPH * nph * 64; }

struct Smem {
  // byte offsets into dynamic LDS
  int codes;  // int8 [MT][K + 16]
  int red;    // int32 [2][kStreamers][64][4] partial tiles, by tile parity
  int wsl;    // float [2][16] weight scales of the tile, by tile parity
  int amax;   // float [kMaxHelpers][kMaxMT] per-helper token maxima
  int qp;     // float [kMaxMT] token scales
  int cnt;    // int: helper wavefronts that published their maxima
  int bytes;
};

__host__ __device__ inline Smem smem_layout(int K, int MT) {
  Smem s;
  s.codes = 0;
  s.red = (MT * (K + 16) + 255) / 256 * 256;
  s.wsl = s.red + 2 * kStreamers * 256 * 4;
  s.amax = s.wsl + 2 * 16 * 4;
  s.qp = s.amax + kMaxHelpers * kMaxMT * 4;
  s.cnt = s.qp + kMaxMT * 4;
  s.bytes = s.cnt + 16;
  return s;
}

// Streamer role: stream this workgroup's tiles through MFMA against the LDS
// code matrix and hand each tile's partial 16x16 sums (and, from wavefront 0,
// the weight scales) to the helpers.  Units (u = phase u % NPH of the
// workgroup's tile u / NPH) rotate through NBUF register buffers; as NBUF
// divides NPH, a tile's last phase always lands in the last buffer, whose
// issue also fetches the tile's weight scales.  The loop holds only this
// role's loads, all issued unconditionally (out-of-range offsets read zero
// without touching memory), so the compiler's in-order wait counts stay exact.
template <int MT, int NPH, int NBUF>
__device__ __forceinline__ void streamer(const int8_t* __restrict__ wq,
                                         const float* __restrict__ wscale, int N, int K,
                                         int first, int G, int T, int wave, int lane,
                                         const int8_t* codes, int Ks, int32_t* red, float* wsl) {
  static_assert(NPH % NBUF == 0, "a tile's last phase must land in the last buffer");
  const int r = lane & 15, g = lane >> 4;
  const int nch = (K + 63) >> 6;
  const int cw = wave * (NPH * kPH);  // first chunk of this wavefront
  v4i a[NBUF][kPH];
  float wsv = 0.0f;  // wavefront 0, lanes 0..15: weight scale of the tile in the last buffer

  auto issue = [&](v4i (&a)[kPH], int u, bool second) {
    const int t = u / NPH, ph = u - t * NPH;
    const bool valid = t < T;
    const int tile = first + (valid ? t : 0) * G;
    const buffer_rsrc rs =
        make_rsrc(wq + (size_t)tile * nch * 1024, valid ? (uint32_t)nch * 1024u : 0u);
#pragma unroll
    for (int j = 0; j < kPH; ++j) {
      const int c = cw + ph * kPH + j;
      a[j] = load16<kNonTemporal>(rs, c < nch ? c * 1024 + lane * 16 : kOutOfRange);
    }
    if (second) {
      const int rows = (valid && ph == NPH - 1) ? min(16, N - tile * 16) : 0;
      const buffer_rsrc ss = make_rsrc(wscale + (size_t)tile * 16, (uint32_t)rows * 4u);
      wsv = __int_as_float(load4(ss, (wave == 0 && lane < 16) ? lane * 4 : kOutOfRange));
    }
  };

  __syncthreads();  // (1) the helpers' activation loads are queued first
#pragma unroll
  for (int b = 0; b < NBUF; ++b) issue(a[b], b, b == NBUF - 1);
  __syncthreads();  // (2) code matrix complete

  const int8_t* brow = codes + (r < MT ? r : 0) * Ks;
  auto bfrag = [&](int c) -> v4i {
    const int k = c * 64 + g * 16;
    const bool ok = r < MT && k < K;
    const v4i v = *reinterpret_cast<const v4i*>(brow + (ok ? k : 0));
    return ok ? v : (v4i){0, 0, 0, 0};
  };
  v4i acc = {0, 0, 0, 0};
  const int units = T * NPH;
  for (int u = 0; u < units; u += NBUF) {
    const int t = u / NPH, ph = u - t * NPH;  // tile and phase of buffer 0
#pragma unroll
    for (int b = 0; b < NBUF; ++b) {
#pragma unroll
      for (int j = 0; j < kPH; ++j)
        acc = mfma_i8_16x16x64(a[b][j], bfrag(cw + (ph + b) * kPH + j), acc);
      if (b < NBUF - 1) {
        issue(a[b], u + b + NBUF, false);
      } else {
        const bool last = ph + b == NPH - 1;
        const int buf = t & 1;
        if (last) {
          // publish before the next issue overwrites wsv: a loop-carried copy of
          // a register with a load in flight would wait for the whole queue
          *reinterpret_cast<v4i*>(red + (buf * kStreamers + wave) * 256 + lane * 4) = acc;
          if (wave == 0 && lane < 16) wsl[buf * 16 + lane] = wsv;
        }
        issue(a[b], u + b + NBUF, true);
        if (last) {
          acc = (v4i){0, 0, 0, 0};
          __syncthreads();  // partials of tile t published
        }
      }
    }
  }
}

// Helper role: smooth and quantize the activation rows into the LDS code
// matrix, then finish every tile: sum the streamers' partials (exact INT32) and
// dequantize to BF16.
template <int MT, int NH, int UP>
__device__ __forceinline__ void helper(const uint16_t* __restrict__ x, const float* __restrict__ s,
                                       int M, int N, int K, int first, int G, int T, int ht,
                                       int hwave, int lane, int8_t* codes, int Ks,
                                       const int32_t* red, const float* wsl, float* amax_part,
                                       float* qp, int* cnt, uint16_t* __restrict__ y,
                                       int32_t* __restrict__ acc_out) {
  constexpr int HT = 64 * NH;  // helper threads
  const int units = K >> 3;    // pieces of 8 K positions per token row
  v4i xv[UP][MT];
  v4i sv[UP][2];
  {
    const buffer_rsrc xrs = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
    const buffer_rsrc srs = make_rsrc(s, (uint32_t)K * 4u);
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const int q = ht + u * HT;
      const bool ok = q < units;
      sv[u][0] = load16(srs, ok ? q * 32 : kOutOfRange);
      sv[u][1] = load16(srs, ok ? q * 32 + 16 : kOutOfRange);
#pragma unroll
      for (int m = 0; m < MT; ++m) xv[u][m] = load16(xrs, ok ? (m * K + q * 8) * 2 : kOutOfRange);
    }
  }
  __syncthreads();  // (1)

  // Per-token absmax of xs = RN32(x * s).  Small windows keep the products in
  // registers for the quantizer; larger ones keep only the loaded operands and
  // form the (deterministic) products again.  Rows m >= M and pieces past K
  // read as zero and contribute nothing.
  constexpr bool kKeepXs = MT * UP <= 12;
  float xs[kKeepXs ? UP : 1][kKeepXs ? MT : 1][8];
  {
    float amax[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) amax[m] = 0.0f;
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      const float sf[8] = {__int_as_float(sv[u][0].x), __int_as_float(sv[u][0].y),
                           __int_as_float(sv[u][0].z), __int_as_float(sv[u][0].w),
                           __int_as_float(sv[u][1].x), __int_as_float(sv[u][1].y),
                           __int_as_float(sv[u][1].z), __int_as_float(sv[u][1].w)};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const uint32_t w4[4] = {(uint32_t)xv[u][m].x, (uint32_t)xv[u][m].y, (uint32_t)xv[u][m].z,
                                (uint32_t)xv[u][m].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
          const float v = bf16_to_f32(bits) * sf[e];
          if (kKeepXs) xs[kKeepXs ? u : 0][kKeepXs ? m : 0][e] = v;
          amax[m] = fmaxf(amax[m], fabsf(v));
        }
      }
    }
    if (!kKeepXs) {
      // opaque copies: the products above must not stay live until the quantizer
#pragma unroll
      for (int u = 0; u < UP; ++u) {
        asm volatile("" : "+v"(sv[u][0]), "+v"(sv[u][1]));
#pragma unroll
        for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(xv[u][m]));
      }
    }
    float wmax[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) wmax[m] = wave_max_nonneg(amax[m]);
    if (lane == 0) {
#pragma unroll
      for (int m = 0; m < MT; ++m) amax_part[hwave * kMaxMT + m] = wmax[m];
      __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
  // Wait for the other helpers' maxima without a workgroup barrier: the
  // streamers are stalled issuing weight loads and must not gate this.  All
  // helpers are resident in this workgroup and publish unconditionally, so the
  // count is reached; the spin is bounded all the same.
  for (int spin = 0; spin < (1 << 22); ++spin) {
    if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= NH) break;
    __builtin_amdgcn_s_sleep(1);
  }
  // every helper forms the row parameters itself: lane m holds row m's
  float row_amax = 0.0f;
  if (lane < MT) {
#pragma unroll
    for (int w = 0; w < NH; ++w) row_amax = fmaxf(row_amax, amax_part[w * kMaxMT + lane]);
  }
  const QParams lp = row_qparams(row_amax);
  if (hwave == 0 && lane < MT) qp[lane] = lp.scale;  // read back by this wavefront's epilogue
  float inv_row[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m)
    inv_row[m] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lp.inv), m));

#pragma unroll
  for (int u = 0; u < UP; ++u) {
    const int q = ht + u * HT;
    if (q < units) {
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float sf[8] = {__int_as_float(sv[u][0].x), __int_as_float(sv[u][0].y),
                             __int_as_float(sv[u][0].z), __int_as_float(sv[u][0].w),
                             __int_as_float(sv[u][1].x), __int_as_float(sv[u][1].y),
                             __int_as_float(sv[u][1].z), __int_as_float(sv[u][1].w)};
        const uint32_t w4[4] = {(uint32_t)xv[u][m].x, (uint32_t)xv[u][m].y, (uint32_t)xv[u][m].z,
                                (uint32_t)xv[u][m].w};
        uint32_t cb[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
          const float v =
              kKeepXs ? xs[kKeepXs ? u : 0][kKeepXs ? m : 0][e] : bf16_to_f32(bits) * sf[e];
          cb[e] = quant_code_biased(v, inv_row[m]);
        }
        uint2 pk;
        pk.x = pack4_low_bytes(cb[0], cb[1], cb[2], cb[3]);
        pk.y = pack4_low_bytes(cb[4], cb[5], cb[6], cb[7]);
        *reinterpret_cast<uint2*>(codes + m * Ks + q * 8) = pk;
      }
    }
  }
  __syncthreads();  // (2)

  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    __syncthreads();  // partials of tile t published
    if (ht < 64) {
      const int tile = first + t * G;
      const int tt = ht & 15;
      const int n0 = tile * 16 + 4 * (ht >> 4);
      if (tt < M && n0 < N) {
        v4i tot = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < kStreamers; ++w)
          tot += *reinterpret_cast<const v4i*>(red + (buf * kStreamers + w) * 256 + ht * 4);
        const float sxt = qp[tt];
        const int tv[4] = {tot.x, tot.y, tot.z, tot.w};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = (float)tv[i];  // round to nearest even
          v = v * sxt;
          v = v * wsl[buf * 16 + 4 * (ht >> 4) + i];
          o[i] = f32_to_bf16_rne(v);
        }
        uint16_t* yr = y + (size_t)tt * N;
        if (n0 + 3 < N && ((reinterpret_cast<uintptr_t>(yr + n0) & 7) == 0)) {
          uint2 pk;
          pk.x = o[0] | (o[1] << 16);
          pk.y = o[2] | (o[3] << 16);
          *reinterpret_cast<uint2*>(yr + n0) = pk;
        } else {
          for (int i = 0; i < 4 && n0 + i < N; ++i) yr[n0 + i] = (uint16_t)o[i];
        }
        if (acc_out)
          for (int i = 0; i < 4 && n0 + i < N; ++i) acc_out[(size_t)tt * N + n0 + i] = tv[i];
      }
    }
  }
}

// The two roles run as separate wavefront-uniform branches.  Both execute the
// same sequence of workgroup barriers: two in the prologue, then one per tile
// (the streamers after writing a tile's partials, the helpers before reading
// them).  The partial-sum buffers are double-buffered by tile parity: a buffer
// is rewritten two tiles later, after the helpers have passed the barrier of
// the tile in between, i.e. after they finished reading it.
template <int MT, int NPH>
__global__ __launch_bounds__(64 * (kStreamers + variant_nh(NPH))) void w8a8_linear_fused_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ s, const int8_t* __restrict__ wq,
    const float* __restrict__ wscale, int M, int N, int K, int tiles, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out) {
  constexpr int NH = variant_nh(NPH);
  constexpr int UP = variant_up(NPH);
  extern __shared__ __align__(16) char smem[];
  const Smem L = smem_layout(K, MT);
  int8_t* codes = reinterpret_cast<int8_t*>(smem + L.codes);
  int32_t* red = reinterpret_cast<int32_t*>(smem + L.red);
  float* wsl = reinterpret_cast<float*>(smem + L.wsl);
  float* amax_part = reinterpret_cast<float*>(smem + L.amax);
  float* qp = reinterpret_cast<float*>(smem + L.qp);
  int* cnt = reinterpret_cast<int*>(smem + L.cnt);
  const int Ks = K + 16;  // padded LDS row: spreads the token rows over the banks

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  if (tid == 0) *cnt = 0;  // ordered before use by the first barrier
  const int G = gridDim.x;
  const int first = blockIdx.x;
  const int T = first < tiles ? (tiles - first + G - 1) / G : 0;
  if (T == 0) return;
  if (wave < kStreamers) {
    streamer<MT, NPH, variant_nbuf(NPH)>(wq, wscale, N, K, first, G, T, wave, lane, codes, Ks, red,
                                         wsl);
  } else {
    helper<MT, NH, UP>(x, s, M, N, K, first, G, T, tid - 64 * kStreamers, wave - kStreamers, lane,
                       codes, Ks, red, wsl, amax_part, qp, cnt, y, acc_out);
  }
}

template <int MT, int NPH>
hipError_t launch_variant(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                          const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&w8a8_linear_fused_kernel<MT, NPH>),
      hipFuncAttributeMaxDynamicSharedMemorySize, smem_layout(variant_kmax(NPH), MT).bytes);
  if (attr != hipSuccess) return attr;
  w8a8_linear_fused_kernel<MT, NPH>
      <<<dim3(p.grid), dim3(64 * p.waves), p.lds, st>>>(x, s, wq, w_scale, (int)p.M, (int)p.N,
                                                         (int)p.K, p.tiles, y, acc_out);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                     const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st) {
  switch (p.nph) {
    case 2: return launch_variant<MT, 2>(p, x, s, wq, w_scale, y, acc_out, st);
    case 4: return launch_variant<MT, 4>(p, x, s, wq, w_scale, y, acc_out, st);
    default: return launch_variant<MT, 6>(p, x, s, wq, w_scale, y, acc_out, st);
  }
}

}  // namespace

bool fused_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= kMaxMT && K <= variant_kmax(6);
}

FusedPlan plan_fused(int64_t M, int64_t N, int64_t K) {
  FusedPlan p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.tiles = (int)((N + 15) / 16);
  p.nch = (int)((K + 63) / 64);
  p.mt = M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 6 ? 6 : 8));
  p.nph = K <= variant_kmax(2) ? 2 : (K <= variant_kmax(4) ? 4 : 6);
  p.waves = kStreamers + variant_nh(p.nph);
  p.lds = smem_layout((int)K, p.mt).bytes;
  const int cap = kNumCU;  // one persistent workgroup per compute unit
  p.grid = p.tiles < cap ? p.tiles : cap;
  return p;
}

const char* fused_kernel_name(const FusedPlan& p) {
  static const char* const names[4][3] = {
      {"w8a8_linear_fused_kernel<2, 2>", "w8a8_linear_fused_kernel<2, 4>",
       "w8a8_linear_fused_kernel<2, 6>"},
      {"w8a8_linear_fused_kernel<4, 2>", "w8a8_linear_fused_kernel<4, 4>",
       "w8a8_linear_fused_kernel<4, 6>"},
      {"w8a8_linear_fused_kernel<6, 2>", "w8a8_linear_fused_kernel<6, 4>",
       "w8a8_linear_fused_kernel<6, 6>"},
      {"w8a8_linear_fused_kernel<8, 2>", "w8a8_linear_fused_kernel<8, 4>",
       "w8a8_linear_fused_kernel<8, 6>"}};
  return names[p.mt / 2 - 1][p.nph / 2 - 1];
}

hipError_t launch_fused(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                        const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st) {
  switch (p.mt) {
    case 2: return launch_mt<2>(p, x, s, wq, w_scale, y, acc_out, st);
    case 4: return launch_mt<4>(p, x, s, wq, w_scale, y, acc_out, st);
    case 6: return launch_mt<6>(p, x, s, wq, w_scale, y, acc_out, st);
    default: return launch_mt<8>(p, x, s, wq, w_scale, y, acc_out, st);
  }
}

}  // namespace quasar
