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
//   * a tile is 16 output channels x all of K; workgroup b handles the
//     contiguous tiles [floor(b*tiles/G), floor((b+1)*tiles/G)) (G = grid
//     size), computed as b q + floor(b r / G) with q, r = tiles / G, tiles % G
//     from the host so that every term fits 32 bits: a workgroup
//     streams one contiguous run of weights, which measured ~5% faster on the
//     LM head than tiles G apart.  The 64-bit form of this division cost
//     ~0.4 us per launch.  Measured alternatives: q = tiles / G tiles each
//     plus one for the first tiles % G workgroups was as fast except on the
//     LM head (3% slower); half tiles at the range ends (to balance QKV's 384
//     tiles on 256 workgroups) were no faster, since a load with half its
//     lanes masked costs the memory pipeline as much as a full one; and
//     handing the last quarter of the tiles out from a device counter (the
//     8 XCDs stream at rates up to 25% apart within a launch) was slower on
//     every linear;
//   * wavefronts are specialized.  A compute unit keeps only ~32-64 KB of
//     vector-memory misses in flight, and a wavefront that issues beyond that
//     stalls at issue until data returns.  So S *streamer* wavefronts own the
//     weight stream, in NPH phases of 8 chunks of 64 K positions per tile:
//     phase p of streamer w is chunks p*8S + 8w .. p*8S + 8w + 7, so a phase
//     of all streamers is one contiguous K range.  Phases rotate through NBUF
//     register buffers (later phases are in flight while earlier ones are
//     multiplied).
//     Each chunk is one
//     contiguous 1 KB of the tile-packed weights (one 128-bit load per lane,
//     already in MFMA A-operand order), loaded with the streaming (nt) policy.
//     Stalling at issue costs a streamer nothing;
//   * NH *helper* wavefronts quantize the activations and finish the tiles.
//     They load the activations first (a barrier orders these loads before
//     any weight load of the compute unit: loads return in issue order), form
//     xs = RN32(x * s), reduce the per-token absmax (DPP within a wavefront,
//     then an LDS counter among the helpers -- not a workgroup barrier, which
//     would wait for the stalled streamers) and write the INT8 codes into an
//     LDS matrix that feeds the MFMA B operand, in K order, announcing each
//     finished K range on an LDS counter: the streamers start multiplying a
//     phase as soon as its codes exist.  Helpers issue no load behind the
//     weight stream;
//   * per tile the streamers' 16x16 INT32 partials (and the tile's weight
//     scales, fetched by streamer 0 with its last phase) go to LDS, and 64
//     helper threads apply the dequant epilogue, 4 channels (8 bytes) per
//     store.
#include <float.h>
#include <limits.h>

#include "quasar_device.hpp"
#include "quasar_internal.hpp"
#include "quasar_sync.hpp"

namespace quasar {
namespace {

constexpr int kMaxMT = 8;          // token rows the one-launch kernel handles
constexpr int kPH = 8;             // chunks per weight phase (8 KB per wavefront)
constexpr int kMaxHelpers = 8;

// Variants by K: S streamer wavefronts with NPH phases per tile each, rotating
// through NBUF register buffers; NH helper wavefronts with UP activation pieces
// (8 K positions) per thread and token row.  The last column is the weight
// bytes a compute unit requests before the code matrix exists: a larger K
// means a longer quantization prologue, which the requested bytes must cover.
//   variant  K        S  NPH NBUF  NH  UP  waves  requested
//   0        <= 4096  4   2   2     8   1   12     64 KB (the whole tile)
//   1        <= 8192  4   4   2     8   2   12     64 KB
//   2        <= 12288 4   6   3     8   3   12     96 KB
// Variant 0 ran 4 helpers with 2 pieces each before; 8 with one piece measured
// faster at every token count: per launch the LM head 2.5-3.8 us, gate_up
// 0.15-0.25 us, QKV and O up to 0.1 us (at 7 and 8 tokens O 0.5 us), QKV at
// 6 tokens +0.09 us.
// NBUF divides NPH, so phase p of every tile uses buffer p % NBUF.
template <int V>
struct Variant {
  static constexpr int S = 4;
  static constexpr int NPH = V == 0 ? 2 : (V == 1 ? 4 : 6);
  static constexpr int NBUF = V == 2 ? 3 : 2;
  static constexpr int NH = 8;
  static constexpr int UP = V == 0 ? 1 : (V == 1 ? 2 : 3);
  static constexpr int KMAX = S * NPH * kPH * 64;
  static constexpr int WAVES = S + NH;
};
static_assert(Variant<0>::KMAX == 4096 && Variant<1>::KMAX == 8192 && Variant<2>::KMAX == 12288,
              "variant K ranges");
static_assert(Variant<0>::NH * 64 * Variant<0>::UP * 8 >= Variant<0>::KMAX &&
                  Variant<1>::NH * 64 * Variant<1>::UP * 8 >= Variant<1>::KMAX &&
                  Variant<2>::NH * 64 * Variant<2>::UP * 8 >= Variant<2>::KMAX,
              "helpers cover K");
static_assert(Variant<0>::UP <= 4 && Variant<1>::UP <= 4 && Variant<2>::UP <= 4,
              "one readiness counter per quantization step");

struct Smem {
  // byte offsets into dynamic LDS
  int codes;  // int8 [MT][K + 16]
  int red;    // int32 [2][S][64][4] partial tiles, by tile parity
  int wsl;    // float [2][16] weight scales of the tile, by tile parity
  int amax;   // float [kMaxHelpers][kMaxMT] per-helper token maxima
  int qp;     // float [kMaxMT] token scales
  int cnt;    // int: helper wavefronts that published their maxima
  int ready;  // int [4]: per quantization step, helper wavefronts that completed it
  int bytes;
};

__host__ __device__ inline Smem smem_layout(int K, int MT, int S) {
  Smem s;
  s.codes = 0;
  s.red = (MT * (K + 16) + 64 + 255) / 256 * 256;  // B reads reach 48 bytes past row MT-1
  s.wsl = s.red + 2 * S * 256 * 4;
  s.amax = s.wsl + 2 * 16 * 4;
  s.qp = s.amax + kMaxHelpers * kMaxMT * 4;
  s.cnt = s.qp + kMaxMT * 4;
  s.ready = s.cnt + 16;
  s.bytes = s.ready + 4 * 4;
  return s;
}

// Streamer role: stream this workgroup's tiles through MFMA against the LDS
// code matrix and hand each tile's partial 16x16 sums (and, from wavefront 0,
// the weight scales) to the helpers.  Units (u = phase u % NPH of the
// workgroup's tile u / NPH) rotate through NBUF register buffers; each buffer's
// issue also fetches the weight scales of its tile when the unit is the tile's
// last phase (zero otherwise), into a register of that buffer.  The loop holds
// only this role's loads, all issued unconditionally (out-of-range offsets read
// zero without touching memory), so the compiler's in-order wait counts stay
// exact.  Units past the last tile are issued (as zero reads) but never
// consumed, and only real tiles take the per-tile barrier, so the barrier
// count matches the helpers'.
template <int MT, int S, int NPH, int NBUF, int NH>
__device__ __forceinline__ void streamer(const int8_t* __restrict__ wq,
                                         const float* __restrict__ wscale, int N, int K,
                                         int first, int T, int wave, int lane,
                                         const int8_t* codes, int Ks, int32_t* red, float* wsl,
                                         const int* ready, const WaitCtl& wc) {
  static_assert(NPH % NBUF == 0, "phase p of every tile uses buffer p % NBUF");
  // helper quantization step u covers K positions [u * 512 NH, (u + 1) * 512 NH):
  // PPS = NH / 4 phases of 8S chunks of 64
  constexpr int PPS = NH * 512 / (S * kPH * 64);
  static_assert(PPS * S * kPH * 64 == NH * 512, "a quantization step covers whole phases");
  const int r = lane & 15, g = lane >> 4;
  const int nch = (K + 63) >> 6;
  const int cw = wave * kPH;  // chunk of phase 0 of this wavefront; phase p adds p * 8S
  v4i a[NBUF][kPH];
  float wsv[NBUF];  // wavefront 0, lanes 0..15: weight scales if the buffer holds a last phase

  // One scalar buffer descriptor per tile (size 0 past the last tile) and the
  // chunk in the vector offset: chunks past K fall outside the tile's range
  // and read zeros without touching memory.  (A descriptor per chunk needed
  // 32 scalar registers per issue, and at K > 4096 the compiler spilled
  // scalars into vector lanes.)
  const int voff = lane * 16;
  auto issue = [&](int b, int tile, int ph) {  // tile < 0: nothing left, read zeros
    const bool valid = tile >= 0;
    const int tl = valid ? tile : 0;
    const buffer_rsrc rs =
        make_rsrc(wq + (size_t)tl * nch * 1024, valid ? (uint32_t)nch * 1024u : 0u);
    const int pbase = voff + (cw + ph * (S * kPH)) * 1024;
#pragma unroll
    for (int j = 0; j < kPH; ++j) a[b][j] = load16<kNonTemporal>(rs, pbase + j * 1024);
    const int rows = (valid && ph == NPH - 1) ? min(16, N - tl * 16) : 0;
    const buffer_rsrc ss = make_rsrc(wscale + (size_t)tl * 16, (uint32_t)rows * 4u);
    wsv[b] = __int_as_float(load4(ss, (wave == 0 && lane < 16) ? lane * 4 : kOutOfRange));
  };

  __syncthreads();  // (1) the helpers' activation loads are queued first
#pragma unroll
  for (int b = 0; b < NBUF; ++b) issue(b, first, b);
  // keep the tile loop from being rotated into the issue above: the in-order
  // wait counts are exact only with the loop entered after all NBUF issues
  __builtin_amdgcn_sched_barrier(0);

  // MFMA B operand: 16 code bytes of token row r at K position 64c + 16g.  No
  // masking is needed: the packed weights are zero past K, so whatever the code
  // rows hold there (and chunks past K, clamped to the last one) multiplies
  // zero, and token columns r >= MT (clamped to row MT - 1) produce outputs the
  // epilogue never stores.
  const int8_t* brow = codes + (r < MT ? r : MT - 1) * Ks + g * 16;
  auto bfrag = [&](int c) -> v4i {
    return *reinterpret_cast<const v4i*>(brow + min(c, nch - 1) * 64);
  };
  // Before a phase of the first tile is multiplied, its codes must exist: per
  // quantization step, the helpers count the wavefronts that finished it (each
  // after its LDS writes have completed), so wait until all NH have finished
  // the step holding this phase.  (One counter per step: a helper with no
  // pieces in a step finishes it at once, so a single running total could
  // reach a step's share while another helper is still writing it.)  The counter orders LDS accesses only, and LDS
  // executes a wavefront's accesses in order, so a relaxed load plus a
  // compiler barrier suffices; an acquire would also wait for this
  // wavefront's weight loads in flight.  All helpers are resident and finish
  // every step unconditionally; the spin is bounded all the same (an expiry
  // is reported in the device status word).
  auto wait_codes = [&](int ph) { lds_wait_at_least(ready + ph / PPS, NH, wc); };
  v4i acc = {0, 0, 0, 0};
  for (int t = 0; t < T; ++t) {
    const int tile = first + t;
    const int next = t + 1 < T ? tile + 1 : -1;
#pragma unroll
    for (int ph = 0; ph < NPH; ++ph) {
      constexpr int kNB = NBUF;
      const int b = ph % kNB;
      if (t == 0 && ph % PPS == 0) wait_codes(ph);
#pragma unroll
      for (int i = 0; i < kPH; ++i)
        acc = mfma_i8_16x16x64(a[b][i], bfrag(cw + ph * (S * kPH) + i), acc);
      // the unit this buffer streams next: a later phase of this tile, or of the next
      const bool same = ph + kNB < NPH;
      const int ntile = same ? tile : next;
      const int nph = same ? ph + kNB : ph + kNB - NPH;
      const bool last = ph == NPH - 1;
      if (last) {
        // publish before the next issue overwrites wsv[b]: a loop-carried copy
        // of a register with a load in flight would wait for the whole queue
        const int buf = t & 1;
        *reinterpret_cast<v4i*>(red + (buf * S + wave) * 256 + lane * 4) = acc;
        if (wave == 0 && lane < 16) wsl[buf * 16 + lane] = wsv[b];
      }
      issue(b, ntile, nph);
      if (last) {
        acc = (v4i){0, 0, 0, 0};
        __syncthreads();  // partials of tile t published
      }
    }
  }
}

// Helper role: smooth and quantize the activation rows into the LDS code
// matrix, then finish every tile: sum the streamers' partials (exact INT32) and
// dequantize to BF16.
template <int MT, int S, int NH, int UP, int kAccShift = 0>
__device__ __forceinline__ void helper(const uint16_t* __restrict__ x, const float* __restrict__ s,
                                       int M, int N, int K, int first, int T, int ht, int hwave,
                                       int lane,
                                       int8_t* codes, int Ks, const int32_t* red, const float* wsl,
                                       float* amax_part, float* qp, int* cnt, int* ready,
                                       uint16_t* __restrict__ y, int32_t* __restrict__ acc_out,
                                       AcceptPartials ap, int G, int swiglu, const WaitCtl& wc) {
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
  lds_wait_at_least(cnt, NH, wc);
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
    // step u (K positions [u * 8 HT, (u + 1) * 8 HT)) of this wavefront is in LDS
    if (lane == 0)
      __hip_atomic_fetch_add(ready + u, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
  }

  // LM-head epilogue: this thread's running (max, lowest argmax, sum of
  // exp((l - max) / T)) over the logits it writes, in increasing channel order
  float am_v = -FLT_MAX, am_s = 0.0f;
  int am_i = INT_MAX;
  auto track = [&](float v, int j) {
    if (v > am_v) {
      if (ap.psum) am_s = am_s * expf((am_v - v) * ap.inv_t) + 1.0f;
      am_v = v;
      am_i = j;
    } else if (ap.psum) {
      am_s += expf((v - am_v) * ap.inv_t);
    }
  };

  for (int t = 0; t < T; ++t) {
    const int tile = first + t;
    const int buf = t & 1;
    __syncthreads();  // partials of tile t published
    if (ht < 64) {
      const int tt = ht & 15;
      const int n0 = tile * 16 + 4 * (ht >> 4);
      if (tt < M && n0 < N) {
        v4i tot = {0, 0, 0, 0};
#pragma unroll
        for (int w = 0; w < S; ++w)
          tot += *reinterpret_cast<const v4i*>(red + (buf * S + w) * 256 + ht * 4);
        const float sxt = qp[tt];
        // the 4-bit streamers accumulate 16x the sums (exact: shift back)
        const int tv[4] = {tot.x >> kAccShift, tot.y >> kAccShift, tot.z >> kAccShift,
                           tot.w >> kAccShift};
        uint32_t o[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v = (float)tv[i];  // round to nearest even
          v = v * sxt;
          v = v * wsl[buf * 16 + 4 * (ht >> 4) + i];
          o[i] = f32_to_bf16_rne(v);
        }
        if (swiglu) {
          // gated weight order: channels 0..7 of the tile are the gate and 8..15
          // the up projections of outputs 8 tile .. + 7; the up values of this
          // thread's 4 outputs sit 32 lanes on.  silu(g) u as quasar_silu_mul:
          // BF16 g and u, binary32 arithmetic, one BF16 rounding.
          uint32_t up[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) up[i] = (uint32_t)__shfl_xor((int)o[i], 32, kWave);
          if ((ht >> 4) < 2) {
            uint32_t a[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float g = bf16_to_f32(o[i]), u = bf16_to_f32(up[i]);
              const float sg = g / (1.0f + expf(-g));
              a[i] = f32_to_bf16_rne(sg * u);
            }
            uint2 pk;
            pk.x = a[0] | (a[1] << 16);
            pk.y = a[2] | (a[3] << 16);
            *reinterpret_cast<uint2*>(y + (size_t)tt * (N / 2) + tile * 8 + 4 * (ht >> 4)) = pk;
          }
          continue;
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
        if (ap.pmax)
          for (int i = 0; i < 4 && n0 + i < N; ++i) track(bf16_to_f32(o[i]), n0 + i);
      }
    }
  }
  if (ap.pmax && ht < 64) {
    // the four threads of token tt are lanes tt, tt + 16, tt + 32, tt + 48
#pragma unroll
    for (int off = 16; off <= 32; off <<= 1) {
      const float ov = __shfl_xor(am_v, off, kWave);
      const int oi = __shfl_xor(am_i, off, kWave);
      const float os = __shfl_xor(am_s, off, kWave);
      const float m = fmaxf(am_v, ov);
      if (ap.psum) am_s = am_s * expf((am_v - m) * ap.inv_t) + os * expf((ov - m) * ap.inv_t);
      if (ov > am_v || (ov == am_v && oi < am_i)) am_i = oi;
      am_v = m;
    }
    if (ht < M) {
      const size_t slot = (size_t)ht * G + blockIdx.x;
      ap.pmax[slot] = am_v;
      ap.pidx[slot] = am_i;
      if (ap.psum) ap.psum[slot] = am_s;
    }
  }
}

// The two roles run as separate wavefront-uniform branches.  Both execute the
// same sequence of workgroup barriers: one in the prologue, then one per tile
// (the streamers after writing a tile's partials, the helpers before reading
// them).  The partial-sum buffers are double-buffered by tile parity: a buffer
// is rewritten two tiles later, after the helpers have passed the barrier of
// the tile in between, i.e. after they finished reading it.
template <int MT, int S, int NPH>
__global__ __launch_bounds__(64 * (S + 8)) void w8a8_linear_fused_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ s, const int8_t* __restrict__ wq,
    const float* __restrict__ wscale, int M, int N, int K, int tq, int tr, int G,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_out, AcceptPartials ap, int swiglu,
    WaitCtl wc) {
  using Var = Variant<NPH == 2 ? 0 : (NPH == 4 ? 1 : 2)>;
  static_assert(Var::S == S && Var::NPH == NPH, "variant");
  extern __shared__ __align__(16) char smem[];
  const Smem L = smem_layout(K, MT, S);
  int8_t* codes = reinterpret_cast<int8_t*>(smem + L.codes);
  int32_t* red = reinterpret_cast<int32_t*>(smem + L.red);
  float* wsl = reinterpret_cast<float*>(smem + L.wsl);
  float* amax_part = reinterpret_cast<float*>(smem + L.amax);
  float* qp = reinterpret_cast<float*>(smem + L.qp);
  int* cnt = reinterpret_cast<int*>(smem + L.cnt);
  int* ready = reinterpret_cast<int*>(smem + L.ready);
  const int Ks = K + 16;  // padded LDS row: spreads the token rows over the banks

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wavefront
  if (tid < 4) {  // ordered before use by the first barrier
    if (tid == 0) *cnt = 0;
    ready[tid] = 0;
  }
  // G (the grid size) <= tiles, so tq >= 1 and every workgroup has a tile;
  // b tq < tiles and b tr < 256 G stay far inside 32 bits
  const int b = blockIdx.x;
  const int first = b * tq + (int)((unsigned int)(b * tr) / (unsigned int)G);
  const int T = (b + 1) * tq + (int)((unsigned int)((b + 1) * tr) / (unsigned int)G) - first;
  if (wave < S) {
    streamer<MT, S, NPH, Var::NBUF, Var::NH>(wq, wscale, N, K, first, T, wave, lane, codes, Ks,
                                             red, wsl, ready, wc);
  } else {
    helper<MT, S, Var::NH, Var::UP>(x, s, M, N, K, first, T, tid - 64 * S, wave - S, lane, codes,
                                    Ks, red, wsl, amax_part, qp, cnt, ready, y, acc_out, ap, G,
                                    swiglu, wc);
  }
}

// ---------------------------------------------------------------------------
// 4-bit weight variant [pt page §5, zh page §5: lower-bit verification named
// as future work].  Same roles, plan and helpers as the kernel above; the
// weights are the 4-bit layout of w4_packed_offset, so each 16-byte load per
// lane carries the A operands of two 64-wide chunks:
//   lo = (v << 4) & 0xF0F0F0F0 (chunk 2c), hi = v & 0xF0F0F0F0 (chunk 2c + 1)
// are each byte's nibble times 16, an exact int8.  The MFMAs then accumulate
// 16x the INT32 sums (|16 acc| <= 16 * 7 * 127 * 12288 < 2^31) and the
// helpers shift the tile's total right by 4.
// Streamer w's phase ph of a tile is packed chunks ph * 8S + 8w .. + 7 (an 8 KB
// run per wavefront, 4096 K positions per phase for the 4 streamers).  Units
// u = tile * NPH4 + phase rotate through NB register buffers, issued NB units
// ahead (across tiles when a tile has one phase).  NB = 2 up to K = 8192; at
// K > 8192 NB = 3 requests the whole 96 KB tile before the longer quantization
// prologue ends (a 4096 x 12288 linear at 6 tokens: 9.9 -> 9.2 us per launch;
// 8 tokens within 0.15 us either way).  Issuing the third buffer only once
// the activations had landed kept half of that gain, and a fourth INT8
// buffer at K > 8192 (128 of the 192 KB tile requested) was 0.9 us slower.
// ---------------------------------------------------------------------------
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

template <int MT, int S, int NPH4, int NH>
__device__ __forceinline__ void streamer_w4(const int8_t* __restrict__ wq4,
                                            const float* __restrict__ wscale, int N, int K,
                                            int first, int T, int wave, int lane,
                                            const int8_t* codes, int Ks, int32_t* red, float* wsl,
                                            const int* ready, const WaitCtl& wc) {
  // three buffers (the whole 96 KB tile) at K > 8192: the stream then waits
  // for the longer quantization prologue with all of its tile requested
  constexpr int NB = NPH4 == 3 ? 3 : 2;
  const int r = lane & 15, g = lane >> 4;
  const int ncp = K >> 7;  // 128-wide pairs of chunks
  const int nch = K >> 6;
  const int U = T * NPH4;
  v4i a[NB][kPH];
  float wsv[NB];
  const int voff = lane * 16;
  auto issue = [&](int b, int u) {  // u >= U: nothing left, read zeros
    const bool valid = u < U;
    const int t = valid ? u / NPH4 : 0;
    const int ph = valid ? u - t * NPH4 : 0;
    const int tl = first + t;
    const int8_t* tbase = wq4 + (size_t)tl * ncp * 1024;
#pragma unroll
    for (int j = 0; j < kPH; ++j) {
      const int pc = ph * (S * kPH) + wave * kPH + j;
      const buffer_rsrc rs =
          make_rsrc(tbase + (size_t)pc * 1024, (valid && pc < ncp) ? 1024u : 0u);
      a[b][j] = load16<kNonTemporal>(rs, voff);
    }
    const int rows = (valid && ph == NPH4 - 1) ? min(16, N - tl * 16) : 0;
    const buffer_rsrc ss = make_rsrc(wscale + (size_t)tl * 16, (uint32_t)rows * 4u);
    wsv[b] = __int_as_float(load4(ss, (wave == 0 && lane < 16) ? lane * 4 : kOutOfRange));
  };

  __syncthreads();  // (1) the helpers' activation loads are queued first
#pragma unroll
  for (int b = 0; b < NB; ++b) issue(b, b);
  __builtin_amdgcn_sched_barrier(0);

  const int8_t* brow = codes + (r < MT ? r : MT - 1) * Ks + g * 16;
  auto bfrag = [&](int c) -> v4i {
    return *reinterpret_cast<const v4i*>(brow + min(c, nch - 1) * 64);
  };
  // the codes of phase ph's K range exist once every helper has finished the
  // quantization step holding its last position (helpers finish steps in order)
  auto wait_codes = [&](int ph) {
    const int kend = min(K, (ph + 1) * S * kPH * 128) - 1;
    lds_wait_at_least(ready + kend / (512 * NH), NH, wc);
  };
  const v4u hi_mask = {0xF0F0F0F0u, 0xF0F0F0F0u, 0xF0F0F0F0u, 0xF0F0F0F0u};
  v4i acc = {0, 0, 0, 0};
  for (int ub = 0; ub < U; ub += NB) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const int u = ub + b;
      const bool live = u < U;
      const int t = u / NPH4;
      const int ph = u - t * NPH4;
      const bool last = live && ph == NPH4 - 1;
      if (live) {
        if (t == 0) wait_codes(ph);
#pragma unroll
        for (int j = 0; j < kPH; ++j) {
          const int pc = ph * (S * kPH) + wave * kPH + j;
          const v4u v = __builtin_bit_cast(v4u, a[b][j]);
          const v4i lo = __builtin_bit_cast(v4i, (v << 4u) & hi_mask);
          const v4i hi = __builtin_bit_cast(v4i, v & hi_mask);
          acc = mfma_i8_16x16x64(lo, bfrag(2 * pc), acc);
          acc = mfma_i8_16x16x64(hi, bfrag(2 * pc + 1), acc);
        }
        if (last) {
          const int buf = t & 1;
          *reinterpret_cast<v4i*>(red + (buf * S + wave) * 256 + lane * 4) = acc;
          if (wave == 0 && lane < 16) wsl[buf * 16 + lane] = wsv[b];
        }
      }
      issue(b, u + NB);
      if (last) {
        acc = (v4i){0, 0, 0, 0};
        __syncthreads();  // partials of tile t published
      }
    }
  }
}

template <int MT, int S, int NPH4>
__global__ __launch_bounds__(64 * (S + 8)) void w4a8_linear_fused_kernel(
    const uint16_t* __restrict__ x, const float* __restrict__ s, const int8_t* __restrict__ wq4,
    const float* __restrict__ wscale, int M, int N, int K, int tq, int tr, int G,
    uint16_t* __restrict__ y, int32_t* __restrict__ acc_out, WaitCtl wc) {
  using Var = Variant<NPH4 == 1 ? 0 : (NPH4 == 2 ? 1 : 2)>;
  static_assert(Var::S == S && Var::NPH == 2 * NPH4, "variant");
  extern __shared__ __align__(16) char smem[];
  const Smem L = smem_layout(K, MT, S);
  int8_t* codes = reinterpret_cast<int8_t*>(smem + L.codes);
  int32_t* red = reinterpret_cast<int32_t*>(smem + L.red);
  float* wsl = reinterpret_cast<float*>(smem + L.wsl);
  float* amax_part = reinterpret_cast<float*>(smem + L.amax);
  float* qp = reinterpret_cast<float*>(smem + L.qp);
  int* cnt = reinterpret_cast<int*>(smem + L.cnt);
  int* ready = reinterpret_cast<int*>(smem + L.ready);
  const int Ks = K + 16;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 4) {
    if (tid == 0) *cnt = 0;
    ready[tid] = 0;
  }
  const int b = blockIdx.x;
  const int first = b * tq + (int)((unsigned int)(b * tr) / (unsigned int)G);
  const int T = (b + 1) * tq + (int)((unsigned int)((b + 1) * tr) / (unsigned int)G) - first;
  if (wave < S) {
    streamer_w4<MT, S, NPH4, Var::NH>(wq4, wscale, N, K, first, T, wave, lane, codes, Ks, red,
                                      wsl, ready, wc);
  } else {
    helper<MT, S, Var::NH, Var::UP, 4>(x, s, M, N, K, first, T, tid - 64 * S, wave - S, lane,
                                      codes, Ks, red, wsl, amax_part, qp, cnt, ready, y, acc_out,
                                      AcceptPartials{nullptr, nullptr, nullptr, 0.0f}, G, 0, wc);
  }
}

template <int MT, int NPH4>
hipError_t launch_w4(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq4,
                     const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st) {
  constexpr int S = 4;
  auto kernel = &w4a8_linear_fused_kernel<MT, S, NPH4>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          smem_layout(Variant<NPH4 - 1>::KMAX, MT, S).bytes);
  if (attr != hipSuccess) return attr;
  const WaitCtl wc = wait_ctl_for_current_device();
  if (!wc.status) return hipErrorInvalidSymbol;
  kernel<<<dim3(p.grid), dim3(64 * (S + 8)), p.lds, st>>>(
      x, s, wq4, w_scale, (int)p.M, (int)p.N, (int)p.K, p.tiles / p.grid, p.tiles % p.grid,
      p.grid, y, acc_out, wc);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_w4_mt(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq4,
                        const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st) {
  switch (p.variant) {
    case 0: return launch_w4<MT, 1>(p, x, s, wq4, w_scale, y, acc_out, st);
    case 1: return launch_w4<MT, 2>(p, x, s, wq4, w_scale, y, acc_out, st);
    default: return launch_w4<MT, 3>(p, x, s, wq4, w_scale, y, acc_out, st);
  }
}

template <int MT, int V>
hipError_t launch_variant(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                          const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st,
                          const AcceptPartials& ap, int swiglu) {
  using Var = Variant<V>;
  auto kernel = &w8a8_linear_fused_kernel<MT, Var::S, Var::NPH>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          smem_layout(Var::KMAX, MT, Var::S).bytes);
  if (attr != hipSuccess) return attr;
  const WaitCtl wc = wait_ctl_for_current_device();
  if (!wc.status) return hipErrorInvalidSymbol;
  kernel<<<dim3(p.grid), dim3(64 * Var::WAVES), p.lds, st>>>(
      x, s, wq, w_scale, (int)p.M, (int)p.N, (int)p.K, p.tiles / p.grid, p.tiles % p.grid, p.grid,
      y, acc_out, ap, swiglu, wc);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_mt(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                     const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st,
                     const AcceptPartials& ap, int swiglu) {
  switch (p.variant) {
    case 0: return launch_variant<MT, 0>(p, x, s, wq, w_scale, y, acc_out, st, ap, swiglu);
    case 1: return launch_variant<MT, 1>(p, x, s, wq, w_scale, y, acc_out, st, ap, swiglu);
    default: return launch_variant<MT, 2>(p, x, s, wq, w_scale, y, acc_out, st, ap, swiglu);
  }
}

}  // namespace

bool fused_supported(int64_t M, int64_t K) {
  return M >= 1 && M <= kMaxMT && K <= Variant<2>::KMAX;
}

FusedPlan plan_fused(int64_t M, int64_t N, int64_t K) {
  FusedPlan p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.tiles = (int)((N + 15) / 16);
  p.nch = (int)((K + 63) / 64);
  p.mt = M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 6 ? 6 : 8));
  p.variant = K <= Variant<0>::KMAX ? 0 : (K <= Variant<1>::KMAX ? 1 : 2);
  p.waves = p.variant == 0 ? Variant<0>::WAVES
                           : (p.variant == 1 ? Variant<1>::WAVES : Variant<2>::WAVES);
  const int S = p.variant == 2 ? Variant<2>::S : Variant<0>::S;
  p.lds = smem_layout((int)K, p.mt, S).bytes;
  const int cap = kNumCU;  // one persistent workgroup per compute unit
  p.grid = p.tiles < cap ? p.tiles : cap;
  return p;
}

bool w4_supported(int64_t M, int64_t K) {
  return fused_supported(M, K) && K % 128 == 0;
}

const char* fused_w4_kernel_name(const FusedPlan& p) {
  // <token rows, streamer wavefronts, 8 KB phases per streamer and tile>
  static const char* const names[4][3] = {
      {"w4a8_linear_fused_kernel<2, 4, 1>", "w4a8_linear_fused_kernel<2, 4, 2>",
       "w4a8_linear_fused_kernel<2, 4, 3>"},
      {"w4a8_linear_fused_kernel<4, 4, 1>", "w4a8_linear_fused_kernel<4, 4, 2>",
       "w4a8_linear_fused_kernel<4, 4, 3>"},
      {"w4a8_linear_fused_kernel<6, 4, 1>", "w4a8_linear_fused_kernel<6, 4, 2>",
       "w4a8_linear_fused_kernel<6, 4, 3>"},
      {"w4a8_linear_fused_kernel<8, 4, 1>", "w4a8_linear_fused_kernel<8, 4, 2>",
       "w4a8_linear_fused_kernel<8, 4, 3>"}};
  return names[p.mt / 2 - 1][p.variant];
}

hipError_t launch_fused_w4(const FusedPlan& p, const uint16_t* x, const float* s,
                           const int8_t* wq4, const float* w_scale, uint16_t* y, int32_t* acc_out,
                           hipStream_t st) {
  switch (p.mt) {
    case 2: return launch_w4_mt<2>(p, x, s, wq4, w_scale, y, acc_out, st);
    case 4: return launch_w4_mt<4>(p, x, s, wq4, w_scale, y, acc_out, st);
    case 6: return launch_w4_mt<6>(p, x, s, wq4, w_scale, y, acc_out, st);
    default: return launch_w4_mt<8>(p, x, s, wq4, w_scale, y, acc_out, st);
  }
}

const char* fused_kernel_name(const FusedPlan& p) {
  // <token rows, streamer wavefronts, phases per streamer and tile>
  static const char* const names[4][3] = {
      {"w8a8_linear_fused_kernel<2, 4, 2>", "w8a8_linear_fused_kernel<2, 4, 4>",
       "w8a8_linear_fused_kernel<2, 4, 6>"},
      {"w8a8_linear_fused_kernel<4, 4, 2>", "w8a8_linear_fused_kernel<4, 4, 4>",
       "w8a8_linear_fused_kernel<4, 4, 6>"},
      {"w8a8_linear_fused_kernel<6, 4, 2>", "w8a8_linear_fused_kernel<6, 4, 4>",
       "w8a8_linear_fused_kernel<6, 4, 6>"},
      {"w8a8_linear_fused_kernel<8, 4, 2>", "w8a8_linear_fused_kernel<8, 4, 4>",
       "w8a8_linear_fused_kernel<8, 4, 6>"}};
  return names[p.mt / 2 - 1][p.variant];
}

hipError_t launch_fused(const FusedPlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                        const float* w_scale, uint16_t* y, int32_t* acc_out, hipStream_t st,
                        const AcceptPartials* partials, bool swiglu) {
  const AcceptPartials ap = partials ? *partials : AcceptPartials{nullptr, nullptr, nullptr, 0.0f};
  const int sw = swiglu ? 1 : 0;
  switch (p.mt) {
    case 2: return launch_mt<2>(p, x, s, wq, w_scale, y, acc_out, st, ap, sw);
    case 4: return launch_mt<4>(p, x, s, wq, w_scale, y, acc_out, st, ap, sw);
    case 6: return launch_mt<6>(p, x, s, wq, w_scale, y, acc_out, st, ap, sw);
    default: return launch_mt<8>(p, x, s, wq, w_scale, y, acc_out, st, ap, sw);
  }
}

}  // namespace quasar
