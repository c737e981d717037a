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

  // ---- 3. per-token absmax of xs = RN32(x * s)
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
        amax[m] = fmaxf(amax[m], fabsf(bf16_to_f32(bits) * sf[e]));
      }
    }
  }
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const float v = wave_max_nonneg(amax[m]);
    if (lane == 0) amax_part[wave * kMaxMT + m] = v;
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

  // ---- 4. quantize this thread's pieces into the LDS code matrix.  The
  // smoothed products are recomputed from the loaded words (bit-identical)
  // rather than kept live across the barriers: the empty asm hides the
  // equality from the compiler, which would otherwise hold all of them.
#pragma unroll
  for (int u = 0; u < UP; ++u) {
    asm volatile("" : "+v"(sv[u][0]), "+v"(sv[u][1]));
#pragma unroll
    for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(xv[u][m]));
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
          cde[e] = quant_code(bf16_to_f32(bits) * sf[e], inv);
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
  if (p.cfg == 0) return launch_cfg<MT, 8, 8>(p, x, s, wq, w_scale, y, acc_out, st);
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
    p.cfg = 0;  // 8 chunks (one phase) x 8 wavefronts
    p.waves = 8;
    p.ch = 8;
  } else {
    p.cfg = 1;  // 16 chunks (two phases) x 12 wavefronts
    p.waves = 12;
    p.ch = 16;
  }
  p.lds = fused_smem((int)K, p.waves, p.mt).bytes;
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
