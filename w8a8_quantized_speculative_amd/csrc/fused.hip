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
//   * the W wavefronts of a workgroup split K: wavefront w owns chunks
//     [w*CH, (w+1)*CH) of 64 K positions, streamed as CH/8 phases of 8 chunks;
//     each chunk is one contiguous 1 KB of the tile-packed weights (one 128-bit
//     load per lane, already in MFMA A-operand order), loaded with the
//     streaming (nt) cache policy;
//   * the weight registers are double-buffered per phase: the next phase is in
//     flight while the current one is multiplied;
//   * prologue: every wavefront first issues its activation loads, a barrier
//     orders them before any weight load of the compute unit (loads return in
//     issue order, so activations queued behind weights would wait for HBM),
//     then the weight stream starts and the activations are smoothed, reduced
//     to per-token absmax (DPP within wavefronts, LDS across them) and
//     quantized into an LDS code matrix that feeds the MFMA B operand;
//   * per tile the wavefronts' 16x16 INT32 partials are summed in LDS and 64
//     threads apply the dequant epilogue, 4 channels (8 bytes) per store.
#include "quasar_device.hpp"
#include "quasar_internal.hpp"

namespace quasar {
namespace {

constexpr int kMaxMT = 8;  // token rows the one-launch kernel handles
constexpr int kPH = 8;     // chunks per weight phase (8 KB per wavefront)

struct FusedSmem {
  // byte offsets into dynamic LDS
  int codes;  // int8 [MT][K + 16]
  int red;    // int32 [2][W][64][4]
  int amax;   // float [W][kMaxMT]
  int qp;     // float [kMaxMT] (x scale), float [kMaxMT] (inverse)
  int bytes;
};

__host__ __device__ inline FusedSmem fused_smem(int K, int W, int MT) {
  FusedSmem s;
  s.codes = 0;
  s.red = (MT * (K + 16) + 255) / 256 * 256;
  s.amax = s.red + 2 * W * 256 * 4;
  s.qp = s.amax + W * kMaxMT * 4;
  s.bytes = s.qp + 2 * kMaxMT * 4;
  return s;
}

// One phase of one tile for this wavefront: kPH chunks, one contiguous 1 KB
// per chunk.  Chunks past K and units past the workgroup's last one
// (valid == false) read as zero without touching memory, so every call issues
// the same loads and the compiler keeps exact in-order wait counts.  The first
// 64 threads also fetch the 4 weight scales their epilogue needs when this is
// the tile's last phase, so the epilogue never issues a load behind the next
// phase's weight stream.
__device__ __forceinline__ void load_phase(v4i (&a)[kPH], float (&ws)[4], const int8_t* wq,
                                           const float* wscale, bool valid, bool last_phase,
                                           int tile, int N, int nch, int c0, int lane, int tid) {
  const int rows = valid ? min(16, N - tile * 16) : 0;
  const buffer_rsrc rs = make_rsrc(wq + (size_t)(valid ? tile : 0) * nch * 1024,
                                   valid ? (uint32_t)nch * 1024u : 0u);
#pragma unroll
  for (int j = 0; j < kPH; ++j) {
    const int c = c0 + j;
    a[j] = load16<kNonTemporal>(rs, c < nch ? c * 1024 + lane * 16 : kOutOfRange);
  }
  const buffer_rsrc ss = make_rsrc(wscale + (size_t)(valid ? tile : 0) * 16,
                                   (uint32_t)(last_phase ? rows : 0) * 4u);
  const int base = tid < 64 ? 16 * (tid >> 4) : kOutOfRange;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    ws[i] = __int_as_float(load4(ss, base == kOutOfRange ? kOutOfRange : base + 4 * i));
}

// MT token rows, CH chunks per wavefront and tile (CH / kPH phases), W wavefronts.
template <int MT, int CH, int W>
__global__ __launch_bounds__(64 * W) void w8a8_linear_fused_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ s, const int8_t* __restrict__ wq,
    const float* __restrict__ wscale, int M, int N, int K, int tiles, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out) {
  extern __shared__ __align__(16) char smem[];
  constexpr int NT = 64 * W;
  constexpr int NPH = CH / kPH;  // phases per tile
  constexpr int UP = CH / 8;     // prologue pieces (8 K positions) per thread and token row
  // phases issued before the prologue math: both of a two-phase tile when the
  // registers allow, so long rows stream while the prologue runs
  constexpr int PRE = (NPH == 1 || MT <= 6) ? 2 : 1;
  const FusedSmem L = fused_smem(K, W, MT);
  int8_t* codes = reinterpret_cast<int8_t*>(smem + L.codes);
  int32_t* red = reinterpret_cast<int32_t*>(smem + L.red);
  float* amax_part = reinterpret_cast<float*>(smem + L.amax);
  float* qp = reinterpret_cast<float*>(smem + L.qp);
  const int Ks = K + 16;  // padded LDS row: spreads the token rows over the banks

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int nch = (K + 63) >> 6;
  const int cw = wave * CH;  // this wavefront's first chunk
  const int G = gridDim.x;
  const int first = blockIdx.x;
  const int T = first < tiles ? (tiles - first + G - 1) / G : 0;
  if (T == 0) return;
  const int U = T * NPH;  // (tile, phase) units of this workgroup, in order
  auto unit_tile = [&](int u) { return first + (u / NPH) * G; };
  auto unit_c0 = [&](int u) { return cw + (u % NPH) * kPH; };

  // ---- 1. activation loads (8 K positions per piece; rows past M read zero)
  const int units = K >> 3;
  const buffer_rsrc xrs = make_rsrc(x, (uint32_t)M * (uint32_t)K * 2u);
  const buffer_rsrc srs = make_rsrc(s, (uint32_t)K * 4u);
  v4i xv[UP][MT];
  v4i sv[UP][2];
#pragma unroll
  for (int u = 0; u < UP; ++u) {
    const int q = tid + u * NT;
    const bool ok = q < units;
    sv[u][0] = load16(srs, ok ? q * 32 : kOutOfRange);
    sv[u][1] = load16(srs, ok ? q * 32 + 16 : kOutOfRange);
#pragma unroll
    for (int m = 0; m < MT; ++m) xv[u][m] = load16(xrs, ok ? (m * K + q * 8) * 2 : kOutOfRange);
  }
  // every wavefront's activation loads are queued before any weight load
  __syncthreads();

  // ---- 2. the weight stream starts
  v4i a0[kPH], a1[kPH];
  float ws0[4], ws1[4];
  auto issue = [&](v4i (&a)[kPH], float (&ws)[4], int u) {
    load_phase(a, ws, wq, wscale, u < U, u % NPH == NPH - 1, unit_tile(u), N, nch, unit_c0(u),
               lane, tid);
  };
  issue(a0, ws0, 0);
  if (PRE == 2) issue(a1, ws1, 1);
  // keep the scheduler from sinking the weight loads below the prologue math
  // (they do not depend on it, so it otherwise delays the stream by microseconds)
  __builtin_amdgcn_sched_barrier(0);

  // ---- 3. per-token absmax of xs = RN32(x * s).  With one piece per thread
  // the smoothed values stay in registers for the quantize step; with two the
  // registers go to the weight stream and the products are recomputed later.
  constexpr bool kKeepXs = (UP == 1);
  float xs[kKeepXs ? MT : 1][8];
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
        if (kKeepXs) xs[kKeepXs ? m : 0][e] = v;
        amax[m] = fmaxf(amax[m], fabsf(v));
      }
    }
  }
  // wavefront maxima (DPP), then across wavefronts through LDS
  float wmax[MT];
#pragma unroll
  for (int m = 0; m < MT; ++m) wmax[m] = wave_max_nonneg(amax[m]);
  if (lane == 0) {
#pragma unroll
    for (int m = 0; m < MT; ++m) amax_part[wave * kMaxMT + m] = wmax[m];
  }
  __syncthreads();
  if (tid < MT) {
    float v = 0.0f;
    for (int w = 0; w < W; ++w) v = fmaxf(v, amax_part[w * kMaxMT + tid]);
    const QParams p = row_qparams(v);
    qp[tid] = p.scale;
    qp[kMaxMT + tid] = p.inv;
  }
  __syncthreads();

  // ---- 4. quantize this thread's pieces into the LDS code matrix.  Where the
  // smoothed products are recomputed (bit-identical), the empty asm hides the
  // equality from the compiler, which would otherwise keep them all live.
  if (!kKeepXs) {
#pragma unroll
    for (int u = 0; u < UP; ++u) {
      asm volatile("" : "+v"(sv[u][0]), "+v"(sv[u][1]));
#pragma unroll
      for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(xv[u][m]));
    }
  }
#pragma unroll
  for (int u = 0; u < UP; ++u) {
    const int q = tid + u * NT;
    if (q < units) {
      const float sf[8] = {__int_as_float(sv[u][0].x), __int_as_float(sv[u][0].y),
                           __int_as_float(sv[u][0].z), __int_as_float(sv[u][0].w),
                           __int_as_float(sv[u][1].x), __int_as_float(sv[u][1].y),
                           __int_as_float(sv[u][1].z), __int_as_float(sv[u][1].w)};
#pragma unroll
      for (int m = 0; m < MT; ++m) {
        const float inv = qp[kMaxMT + m];
        const uint32_t w4[4] = {(uint32_t)xv[u][m].x, (uint32_t)xv[u][m].y, (uint32_t)xv[u][m].z,
                                (uint32_t)xv[u][m].w};
        int cde[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
          const float v = kKeepXs ? xs[kKeepXs ? m : 0][e] : bf16_to_f32(bits) * sf[e];
          cde[e] = quant_code_in_range(v, inv);
        }
        uint2 pk;
        pk.x = pack4_i8(cde[0], cde[1], cde[2], cde[3]);
        pk.y = pack4_i8(cde[4], cde[5], cde[6], cde[7]);
        *reinterpret_cast<uint2*>(codes + m * Ks + q * 8) = pk;
      }
    }
  }
  __syncthreads();
  if (PRE == 1) issue(a1, ws1, 1);
  __builtin_amdgcn_sched_barrier(0);

  // MFMA B operand of chunk c for this lane: 16 codes of token r at K offset
  // 64c + 16g (zero for rows past MT or K past K), read from LDS.
  const int8_t* brow = codes + (r < MT ? r : 0) * Ks;
  auto bfrag = [&](int c) -> v4i {
    const int k = c * 64 + g * 16;
    const bool ok = r < MT && k < K;
    const v4i v = *reinterpret_cast<const v4i*>(brow + (ok ? k : 0));
    return ok ? v : (v4i){0, 0, 0, 0};
  };

  v4i acc = {0, 0, 0, 0};
  int epi = 0;  // epilogues done (selects the LDS reduction buffer)
  auto consume = [&](const v4i (&a)[kPH], const float (&ws)[4], int u) {
#pragma unroll
    for (int j = 0; j < kPH; ++j) acc = mfma_i8_16x16x64(a[j], bfrag(unit_c0(u) + j), acc);
    if (u % NPH != NPH - 1) return;
    // ---- tile complete: sum the wavefronts' partial tiles, dequantize, store
    const int tile = unit_tile(u);
    int32_t* rb = red + (epi & 1) * (W * 256);
    ++epi;
    *reinterpret_cast<v4i*>(rb + wave * 256 + lane * 4) = acc;
    acc = (v4i){0, 0, 0, 0};
    __syncthreads();
    const int t = tid & 15;
    const int n0 = tile * 16 + 4 * (tid >> 4);
    if (tid < 64 && t < M && n0 < N) {
      v4i tot = {0, 0, 0, 0};
      for (int w = 0; w < W; ++w) tot += *reinterpret_cast<const v4i*>(rb + w * 256 + tid * 4);
      const float sxt = qp[t];
      const int tv[4] = {tot.x, tot.y, tot.z, tot.w};
      uint32_t o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = (float)tv[i];  // round to nearest even
        v = v * sxt;
        v = v * ws[i];
        o[i] = f32_to_bf16_rne(v);
      }
      uint16_t* yr = y + (size_t)t * N;
      if (n0 + 3 < N && ((reinterpret_cast<uintptr_t>(yr + n0) & 7) == 0)) {
        uint2 pk;
        pk.x = o[0] | (o[1] << 16);
        pk.y = o[2] | (o[3] << 16);
        *reinterpret_cast<uint2*>(yr + n0) = pk;
      } else {
        for (int i = 0; i < 4 && n0 + i < N; ++i) yr[n0 + i] = (uint16_t)o[i];
      }
      if (acc_out)
        for (int i = 0; i < 4 && n0 + i < N; ++i) acc_out[(size_t)t * N + n0 + i] = tv[i];
    }
  };

  // ---- 5. steady state: one phase in flight while the other is consumed
  for (int u = 0; u < U; u += 2) {
    consume(a0, ws0, u);
    issue(a0, ws0, u + 2);
    if (u + 1 >= U) break;
    consume(a1, ws1, u + 1);
    issue(a1, ws1, u + 3);
  }
}

// ---------------------------------------------------------------------------
// Wave-specialized variant for K <= 4096 (one 8-wavefront workgroup per CU).
//
// A compute unit only keeps ~32 KB of vector-memory misses in flight; a
// wavefront that issues loads beyond that stalls at issue until earlier data
// returns.  So the roles are split: the four *streamer* wavefronts own all K
// chunks of a tile (16 each, two phases of 8, double-buffered) and do nothing
// but stream weights and issue MFMAs -- stalling at issue costs them nothing --
// while the four *helper* wavefronts quantize the activations (never issuing a
// load behind the weight stream) and run each tile's epilogue.  Streamer 0
// fetches the tile's weight scales with its last phase and hands them to the
// helpers through LDS with the partial sums.
// ---------------------------------------------------------------------------
constexpr int kWsStreamers = 4;
constexpr int kWsHelpers = 4;
constexpr int kWsCH = 16;  // chunks per streamer and tile (K <= 4096)

struct WsSmem {
  int codes;  // int8 [MT][K + 16]
  int red;    // int32 [2][streamers][64][4]
  int wsl;    // float [2][16] weight scales of the tile
  int amax;   // float [helpers][kMaxMT]
  int qp;     // float [kMaxMT] scale
  int cnt;    // int: helper wavefronts that published their absmax
  int bytes;
};

__host__ __device__ inline WsSmem ws_smem(int K, int MT) {
  WsSmem s;
  s.codes = 0;
  s.red = (MT * (K + 16) + 255) / 256 * 256;
  s.wsl = s.red + 2 * kWsStreamers * 256 * 4;
  s.amax = s.wsl + 2 * 16 * 4;
  s.qp = s.amax + kWsHelpers * kMaxMT * 4;
  s.cnt = s.qp + kMaxMT * 4;
  s.bytes = s.cnt + 16;
  return s;
}

// Streamer role: stream this workgroup's tiles (16 chunks per wavefront, two
// double-buffered phases of 8) through MFMA against the LDS code matrix and
// hand each tile's partial 16x16 sums (and, from wavefront 0, the weight
// scales) to the helpers.  The loop holds only this role's loads, so every wait
// count is exact.
template <int MT>
__device__ __forceinline__ void ws_streamer(const int8_t* __restrict__ wq,
                                            const float* __restrict__ wscale, int N, int K,
                                            int first, int G, int T, int wave, int lane,
                                            const int8_t* codes, int Ks, int32_t* red, float* wsl) {
  const int r = lane & 15, g = lane >> 4;
  const int nch = (K + 63) >> 6;
  const int cw = wave * kWsCH;
  v4i a0[kPH], a1[kPH];
  float wsv = 0.0f;  // wavefront 0, lanes 0..15: weight scale of the tile in a1
  auto issue = [&](v4i (&a)[kPH], int t, int phase) {
    const bool valid = t < T;
    const int tile = first + (valid ? t : 0) * G;
    const buffer_rsrc rs =
        make_rsrc(wq + (size_t)tile * nch * 1024, valid ? (uint32_t)nch * 1024u : 0u);
#pragma unroll
    for (int j = 0; j < kPH; ++j) {
      const int c = cw + phase * kPH + j;
      a[j] = load16<kNonTemporal>(rs, c < nch ? c * 1024 + lane * 16 : kOutOfRange);
    }
    if (phase == 1) {
      const int rows = valid ? min(16, N - tile * 16) : 0;
      const buffer_rsrc ss = make_rsrc(wscale + (size_t)tile * 16, (uint32_t)rows * 4u);
      wsv = __int_as_float(load4(ss, (wave == 0 && lane < 16) ? lane * 4 : kOutOfRange));
    }
  };

  __syncthreads();  // (1) the helpers' activation loads are queued first
  issue(a0, 0, 0);
  issue(a1, 0, 1);
  __syncthreads();  // (2) code matrix complete

  const int8_t* brow = codes + (r < MT ? r : 0) * Ks;
  auto bfrag = [&](int c) -> v4i {
    const int k = c * 64 + g * 16;
    const bool ok = r < MT && k < K;
    const v4i v = *reinterpret_cast<const v4i*>(brow + (ok ? k : 0));
    return ok ? v : (v4i){0, 0, 0, 0};
  };
  for (int t = 0; t < T; ++t) {
    const int buf = t & 1;
    v4i acc = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kPH; ++j) acc = mfma_i8_16x16x64(a0[j], bfrag(cw + j), acc);
    issue(a0, t + 1, 0);
#pragma unroll
    for (int j = 0; j < kPH; ++j) acc = mfma_i8_16x16x64(a1[j], bfrag(cw + kPH + j), acc);
    // publish before the next issue overwrites wsv: a loop-carried copy of a
    // register with a load in flight would wait for the whole queue
    *reinterpret_cast<v4i*>(red + (buf * kWsStreamers + wave) * 256 + lane * 4) = acc;
    if (wave == 0 && lane < 16) wsl[buf * 16 + lane] = wsv;
    issue(a1, t + 1, 1);
    __syncthreads();  // partials of tile t published
  }
}

// Helper role: smooth and quantize the activation rows into the LDS code
// matrix, then finish every tile: sum the streamers' partials (exact INT32) and
// dequantize to BF16.  Helpers issue no load after the activations, so nothing
// of theirs queues behind the weight stream.
template <int MT>
__device__ __forceinline__ void ws_helper(const uint16_t* __restrict__ x,
                                          const float* __restrict__ s, int M, int N, int K,
                                          int first, int G, int T, int ht, int hwave, int lane,
                                          int8_t* codes, int Ks, const int32_t* red,
                                          const float* wsl, float* amax_part, float* qp, int* cnt,
                                          uint16_t* __restrict__ y, int32_t* __restrict__ acc_out) {
  constexpr int HT = 64 * kWsHelpers;  // helper threads
  constexpr int UP = 2;                // pieces (8 K positions) per thread and token row
  const int units = K >> 3;
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

  // per-token absmax of xs = RN32(x * s).  Up to six token rows the products
  // stay in registers for the quantizer; wider windows keep only the loaded
  // operands and form the (deterministic) products again.
  constexpr bool kKeepXs = MT <= 6;
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
    if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= kWsHelpers) break;
    __builtin_amdgcn_s_sleep(1);
  }
  // every helper forms the row parameters itself: lane m holds row m's
  float row_amax = 0.0f;
  if (lane < MT) {
#pragma unroll
    for (int w = 0; w < kWsHelpers; ++w) row_amax = fmaxf(row_amax, amax_part[w * kMaxMT + lane]);
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
        const float inv = inv_row[m];
        const float sf[8] = {__int_as_float(sv[u][0].x), __int_as_float(sv[u][0].y),
                             __int_as_float(sv[u][0].z), __int_as_float(sv[u][0].w),
                             __int_as_float(sv[u][1].x), __int_as_float(sv[u][1].y),
                             __int_as_float(sv[u][1].z), __int_as_float(sv[u][1].w)};
        const uint32_t w4[4] = {(uint32_t)xv[u][m].x, (uint32_t)xv[u][m].y, (uint32_t)xv[u][m].z,
                                (uint32_t)xv[u][m].w};
        int cde[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
          const float v =
              kKeepXs ? xs[kKeepXs ? u : 0][kKeepXs ? m : 0][e] : bf16_to_f32(bits) * sf[e];
          cde[e] = quant_code_in_range(v, inv);
        }
        uint2 pk;
        pk.x = pack4_i8(cde[0], cde[1], cde[2], cde[3]);
        pk.y = pack4_i8(cde[4], cde[5], cde[6], cde[7]);
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
        for (int w = 0; w < kWsStreamers; ++w)
          tot += *reinterpret_cast<const v4i*>(red + (buf * kWsStreamers + w) * 256 + ht * 4);
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
template <int MT>
__global__ __launch_bounds__(64 * (kWsStreamers + kWsHelpers)) void w8a8_linear_ws_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ s, const int8_t* __restrict__ wq,
    const float* __restrict__ wscale, int M, int N, int K, int tiles, uint16_t* __restrict__ y,
    int32_t* __restrict__ acc_out) {
  extern __shared__ __align__(16) char smem[];
  const WsSmem L = ws_smem(K, MT);
  int8_t* codes = reinterpret_cast<int8_t*>(smem + L.codes);
  int32_t* red = reinterpret_cast<int32_t*>(smem + L.red);
  float* wsl = reinterpret_cast<float*>(smem + L.wsl);
  float* amax_part = reinterpret_cast<float*>(smem + L.amax);
  float* qp = reinterpret_cast<float*>(smem + L.qp);
  int* cnt = reinterpret_cast<int*>(smem + L.cnt);
  const int Ks = K + 16;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  if (tid == 0) *cnt = 0;  // ordered before use by the first barrier
  const int G = gridDim.x;
  const int first = blockIdx.x;
  const int T = first < tiles ? (tiles - first + G - 1) / G : 0;
  if (T == 0) return;
  if (wave < kWsStreamers) {
    ws_streamer<MT>(wq, wscale, N, K, first, G, T, wave, lane, codes, Ks, red, wsl);
  } else {
    ws_helper<MT>(x, s, M, N, K, first, G, T, tid - 64 * kWsStreamers, wave - kWsStreamers, lane,
                  codes, Ks, red, wsl, amax_part, qp, cnt, y, acc_out);
  }
}

template <int MT>
hipError_t launch_ws(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                     const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st) {
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&w8a8_linear_ws_kernel<MT>),
      hipFuncAttributeMaxDynamicSharedMemorySize, ws_smem(4096, MT).bytes);
  if (attr != hipSuccess) return attr;
  w8a8_linear_ws_kernel<MT><<<dim3(p.grid), dim3(64 * (kWsStreamers + kWsHelpers)), p.lds, st>>>(
      x, s, wq, w_scale, (int)p.M, (int)p.N, (int)p.K, p.tiles, y, acc_out);
  return hipGetLastError();
}

template <int MT, int CH, int W>
hipError_t launch_cfg(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                      const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st) {
  // allow the LDS code matrix of long rows (up to ~123 KB) once per instantiation
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(&w8a8_linear_fused_kernel<MT, CH, W>),
      hipFuncAttributeMaxDynamicSharedMemorySize, fused_smem(12288, W, MT).bytes);
  if (attr != hipSuccess) return attr;
  w8a8_linear_fused_kernel<MT, CH, W><<<dim3(p.grid), dim3(64 * W), p.lds, st>>>(
      x, s, wq, w_scale, (int)p.M, (int)p.N, (int)p.K, p.tiles, y, acc_out);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                     const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st) {
  if (p.cfg == 0) return launch_ws<MT>(p, x, s, wq, w_scale, y, acc_out, st);
  return launch_cfg<MT, 16, 12>(p, x, s, wq, w_scale, y, acc_out, st);
}

}  // namespace

bool fused_supported(int64_t M, int64_t K) { return M >= 1 && M <= kMaxMT && K <= 12288; }

FusedPlan plan_fused(int64_t M, int64_t N, int64_t K) {
  FusedPlan p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.tiles = (int)((N + 15) / 16);
  p.nch = (int)((K + 63) / 64);
  p.mt = M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 6 ? 6 : 8));
  if (p.nch <= 64) {
    p.cfg = 0;  // wave-specialized: 4 streamers x 16 chunks + 4 helpers
    p.waves = 8;
    p.ch = 16;
  } else {
    p.cfg = 1;  // 16 chunks (two phases) x 12 wavefronts
    p.waves = 12;
    p.ch = 16;
  }
  p.lds = p.cfg == 0 ? ws_smem((int)K, p.mt).bytes : fused_smem((int)K, p.waves, p.mt).bytes;
  const int cap = kNumCU;  // one persistent workgroup per compute unit
  p.grid = p.tiles < cap ? p.tiles : cap;
  return p;
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
