// A chain of W8A8 SmoothQuant linears over one verify window (M <= 8 tokens)
// in ONE persistent launch: each link is the verify linear of the small-window
// kernel (online smoothing + dynamic per-token INT8 quantization of the BF16
// input, INT8 x INT8 -> INT32 MFMA product against the resident INT8 weights,
// BF16 dequantization) [Quasar, pt page §2 execution pipeline items 2-4; zh
// page §2 items 2-3], and a link may take as its input the output of an
// earlier link of the same launch.
//
// Why: a verify step runs the target model's linears one after the other,
// each reading the previous one's output, and every one of them streams its
// INT8 weights from HBM [pt page §1: verification is bound by weight loading].
// With one launch per linear, each boundary costs a kernel launch gap, the
// next kernel's start-up, and the time until its activation codes exist --
// all with the weight stream idle.  Here the weight stream does not stop at a
// boundary: a link's weights do not depend on any activation, so the streamer
// wavefronts issue the next link's first weight phases while the current
// link's last tiles are still being multiplied, and the only thing that waits
// for the previous link is the quantization of the next link's input.
//
// Work decomposition: the small-window kernel's, applied link after link.
//   * workgroup b (one per compute unit) owns the contiguous tiles
//     [b q + floor(b r / G), (b + 1) q + floor((b + 1) r / G)) of every link
//     (q, r = tiles / G, tiles % G), 16 output channels x all of K per tile;
//   * S = 4 streamer wavefronts stream the weights in units of one phase (8
//     chunks of 1 KB per wavefront, 2048 K positions for the four) through
//     NBUF register buffers.  The unit sequence runs over (link, tile, phase)
//     across link boundaries, NBUF units ahead of the multiply;
//   * NH = 8 helper wavefronts, per link: wait until the link that writes
//     this link's input is complete in every workgroup, load the BF16 rows and
//     s, form xs = RN32(x * s), reduce the per-token absmax, and write the INT8
//     codes into the LDS code matrix, announcing each 4096-wide K step; then
//     per tile apply the dequant epilogue to the streamers' INT32 partials.
//
// Cross-workgroup protocol (quasar_sync.hpp): workgroup b owns progress word b
// of the workspace's flag header.  It reads it once (`base`); its outputs are
// stored with agent-scope stores, and once they have completed it raises the
// word to base + i + 1.  A link with a dependency waits until every
// workgroup's word has reached base + dep + 1 (one helper wavefront polls) and
// then reads its input with agent-scope loads.  Every workgroup finishes links
// in order, so that means link dep and everything before it is complete.  The grid must be
// resident at once (one workgroup per compute unit); every wait is bounded and
// reported through the device status word if it gives up.
//
// Within a workgroup the code matrix is single-buffered.  A link's codes are
// written only after the helpers have finished the previous link's last tile,
// which the streamers reach only after their last multiply of that link, so
// no reader of the old codes remains.  Every LDS counter only grows: a link's
// targets are offset by the number of links (with tiles) this workgroup has
// already processed.
#include <float.h>
#include <limits.h>

#include "quasar.h"
#include "quasar_device.hpp"
#include "quasar_internal.hpp"
#include "quasar_sync.hpp"

namespace quasar {
namespace {

constexpr int kS = 4;           // streamer wavefronts
constexpr int kNH = 8;          // helper wavefronts
constexpr int kHT = 64 * kNH;   // helper threads
constexpr int kPH = 8;          // 1 KB chunks per streamer and phase
constexpr int kPhaseK = kS * kPH * 64;   // K positions per phase: 2048
constexpr int kStepK = 8 * kHT;          // K positions per quantization step: 4096
constexpr int kUP = kChainMaxK / kStepK; // 8-element pieces per helper thread and row: 3
constexpr int kThreads = 64 * (kS + kNH);
static_assert(kUP * kStepK == kChainMaxK && kUP <= 4, "quantization steps");

struct Smem {
  int codes;  // int8 [MT][K + 16] of the current link
  int red;    // int32 [2][S][64][4] partial tiles, by tile parity
  int wsl;    // float [2][16] weight scales of the tile, by tile parity
  int amax;   // float [NH][8] per-helper token maxima
  int qp;     // float [8] token scales of the current link
  int cnt;    // int: helper wavefronts that published their maxima (grows)
  int ready;  // int [4]: per quantization step, helper wavefronts that completed it (grow)
  int gate;   // int: dependency waits passed (grows)
  int expired;  // int: nonzero once a streamer's wait gave up
  int bytes;
};

__host__ __device__ inline Smem chain_smem(int Kmax, int MT) {
  Smem s;
  s.codes = 0;
  s.red = (MT * (Kmax + 16) + 64 + 255) / 256 * 256;  // B reads reach 48 bytes past row MT-1
  s.wsl = s.red + 2 * kS * 256 * 4;
  s.amax = s.wsl + 2 * 16 * 4;
  s.qp = s.amax + kNH * 8 * 4;
  s.cnt = s.qp + 8 * 4;
  s.ready = s.cnt + 16;
  s.gate = s.ready + 16;
  s.expired = s.gate + 4;
  s.bytes = s.gate + 16;
  return s;
}

// Workgroup b's contiguous tile range of a link with `tiles` tiles.
__device__ __forceinline__ void tile_range(int tiles, int b, int G, int& first, int& T) {
  const int q = tiles / G, r = tiles % G;
  first = b * q + (int)((unsigned)(b * r) / (unsigned)G);
  T = (b + 1) * q + (int)((unsigned)((b + 1) * r) / (unsigned)G) - first;
}

// Position in the streamers' unit sequence (link, tile, phase).  `seq` counts
// the links with tiles in this workgroup before `li`; li == n once exhausted.
struct Cursor {
  int li, seq;
  int tile, tfirst, tend, ph, nph, nch, N, Ks;
  const int8_t* wq;
  const float* ws;
};

__device__ __forceinline__ void cursor_seek(Cursor& c, const quasar_chain_link* __restrict__ links, int n,
                                            int b, int G) {
  while (c.li < n) {
    const quasar_chain_link& L = links[c.li];
    const int N = (int)L.N, K = (int)L.K;
    int first, T;
    tile_range((N + 15) >> 4, b, G, first, T);
    if (T > 0) {
      c.tile = c.tfirst = first;
      c.tend = first + T;
      c.ph = 0;
      c.nch = (K + 63) >> 6;
      c.nph = (K + kPhaseK - 1) / kPhaseK;
      c.N = N;
      c.Ks = K + 16;
      c.wq = L.wq;
      c.ws = L.w_scale;
      return;
    }
    ++c.li;
  }
}

__device__ __forceinline__ void cursor_next(Cursor& c, const quasar_chain_link* __restrict__ links, int n,
                                            int b, int G) {
  if (++c.ph < c.nph) return;
  c.ph = 0;
  if (++c.tile < c.tend) return;
  ++c.li;
  ++c.seq;
  cursor_seek(c, links, n, b, G);
}

// ---------------------------------------------------------------------------
// Streamer role.  Units rotate through NBUF register buffers; each buffer's
// issue also fetches the weight scales of its tile when the unit is the tile's
// last phase (zero otherwise).  All loads are issued unconditionally
// (out-of-range offsets and exhausted units read zero without touching
// memory), so the compiler's in-order wait counts stay exact.
// ---------------------------------------------------------------------------
template <int MT, int NBUF>
__device__ __forceinline__ void chain_streamer(const quasar_chain_link* __restrict__ links, int n, int b, int G,
                                               int wave, int lane, const int8_t* codes,
                                               int32_t* red, float* wsl, const int* ready,
                                               int* expired, const WaitCtl& wc) {
  const int r = lane & 15, g = lane >> 4;
  const int voff = lane * 16;
  v4i a[NBUF][kPH];
  float wsv[NBUF];

  Cursor iss{0, 0, 0, 0, 0, 0, 1, 1, 0, 16, links[0].wq, links[0].w_scale};
  cursor_seek(iss, links, n, b, G);
  Cursor cons = iss;

  auto issue = [&](int bb) {
    const bool valid = iss.li < n;
    const int8_t* tbase = iss.wq + (size_t)(valid ? iss.tile : 0) * iss.nch * 1024;
#pragma unroll
    for (int j = 0; j < kPH; ++j) {
      const int c = iss.ph * (kS * kPH) + wave * kPH + j;
      const buffer_rsrc rs =
          make_rsrc(tbase + (size_t)c * 1024, (valid && c < iss.nch) ? 1024u : 0u);
      a[bb][j] = load16<kNonTemporal>(rs, voff);
    }
    const int rows = (valid && iss.ph == iss.nph - 1) ? min(16, iss.N - iss.tile * 16) : 0;
    const buffer_rsrc ss = make_rsrc(iss.ws + (size_t)(valid ? iss.tile : 0) * 16,
                                     (uint32_t)rows * 4u);
    wsv[bb] = __int_as_float(load4(ss, (wave == 0 && lane < 16) ? lane * 4 : kOutOfRange));
    if (valid) cursor_next(iss, links, n, b, G);
  };

  __syncthreads();  // (1) the helpers' first activation loads are queued first
#pragma unroll
  for (int bb = 0; bb < NBUF; ++bb) issue(bb);
  __builtin_amdgcn_sched_barrier(0);

  // The codes of a phase's K range exist once every helper has finished the
  // quantization step holding it (first tile of a link).  The wait is bounded;
  // an expiry is recorded in LDS and reported by a helper: a global atomic
  // here would make this role's vector-memory count depend on the path, and
  // the compiler's waits before each multiply would no longer be exact.
  auto wait_codes = [&](int step, int target) {
    const int t = target + (int)wc.bias;
    for (int spin = 0;; ++spin) {
      if (__hip_atomic_load(ready + step, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= t)
        break;
      if (spin >= wc.spin_lds) {
        __hip_atomic_store(expired, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    asm volatile("" ::: "memory");
  };

  v4i acc = {0, 0, 0, 0};
  int tcount = 0;  // tiles finished by this workgroup (partial-buffer parity)
  // Every buffer slot issues exactly one unit per pass (zeros once the
  // sequence is exhausted), so the number of loads between a buffer's issue
  // and its use never depends on the path.
  while (cons.li < n) {
#pragma unroll
    for (int bb = 0; bb < NBUF; ++bb) {
      const bool live = cons.li < n;
      bool last = false;
      if (live) {
        if (cons.tile == cons.tfirst && (cons.ph & 1) == 0)
          wait_codes(cons.ph >> 1, kNH * (cons.seq + 1));
        const int8_t* brow = codes + (r < MT ? r : MT - 1) * cons.Ks + g * 16;
#pragma unroll
        for (int i = 0; i < kPH; ++i) {
          const int c = min(cons.ph * (kS * kPH) + wave * kPH + i, cons.nch - 1);
          acc = mfma_i8_16x16x64(a[bb][i], *reinterpret_cast<const v4i*>(brow + c * 64), acc);
        }
        last = cons.ph == cons.nph - 1;
        if (last) {
          // publish before the next issue overwrites wsv[bb]
          const int buf = tcount & 1;
          *reinterpret_cast<v4i*>(red + (buf * kS + wave) * 256 + lane * 4) = acc;
          if (wave == 0 && lane < 16) wsl[buf * 16 + lane] = wsv[bb];
        }
      }
      issue(bb);
      if (live) {
        if (last) {
          acc = (v4i){0, 0, 0, 0};
          ++tcount;
          __syncthreads();  // partials of the tile published
        }
        cursor_next(cons, links, n, b, G);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Helper role.
// ---------------------------------------------------------------------------
template <int MT>
__device__ __forceinline__ void chain_helper(const quasar_chain_link* __restrict__ links, int n,
                                             int M, int b, int G, int ht, int hwave, int lane,
                                             int8_t* codes, const int32_t* red, const float* wsl,
                                             float* amax_part, float* qp, int* cnt, int* ready,
                                             int* gate, const int* expired, uint32_t* progress,
                                             AcceptPartials ap, const WaitCtl& wc) {
  const uint32_t base = load_flag(flag_word(progress, 0, b));
  int qseq = 0;    // links quantized here (LDS counter cnt)
  int dseq = 0;    // dependency waits passed (LDS counter gate)
  int tcount = 0;  // tiles finished (partial-buffer parity)
  bool started = false;  // barrier (1) passed

  for (int li = 0; li < n; ++li) {
    const quasar_chain_link& L = links[li];
    const int N = (int)L.N, K = (int)L.K;
    int first, T;
    tile_range((N + 15) >> 4, b, G, first, T);
    const bool lm_partials = ap.pmax != nullptr && li == n - 1;
    const bool dependent = L.dep >= 0;
    // the next link reads this link's output within this launch
    const bool consumed = li + 1 < n && links[li + 1].dep == li;
    const bool swiglu = (L.flags & QUASAR_LINK_SWIGLU) != 0;
    const int Ks = K + 16;

    if (T > 0) {
      // The first link with tiles that needs no earlier link issues its loads
      // before barrier (1), ahead of every weight load of the compute unit.
      if (!started && dependent) {
        __syncthreads();  // (1)
        started = true;
      }
      if (dependent) {
        // every workgroup has stored its part of the previous link (and its
        // stores have completed) once its progress word has reached base + li
        if (hwave == 0) {
          const uint32_t target = base + (uint32_t)li + wc.bias;
          bool ok = false;
          for (int spin = 0;; ++spin) {
            bool all = true;
            for (int c = lane; c < G; c += 64) all &= reached(load_flag(flag_word(progress, 0, c)), target);
            if (__builtin_amdgcn_ballot_w64(!all) == 0) {
              ok = true;
              break;
            }
            if (spin >= wc.spin_global) break;
            __builtin_amdgcn_s_sleep(1);
          }
          if (!ok && lane == 0) note_expired(wc, kWaitChain);
          after_poll();
          if (lane == 0)
            __hip_atomic_fetch_add(gate, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        } else {
          lds_wait_at_least(gate, dseq + 1, wc);
        }
        ++dseq;
      }
      // smooth and quantize the link's BF16 input (written in this launch for a
      // dependent link: agent-scope loads)
      const int units = K >> 3;  // pieces of 8 K positions per token row
      const int up = (units + kHT - 1) / kHT;
      v4i xv[kUP][MT];
      v4i sv[kUP][2];
      {
        const int64_t ldx = L.ldx;
        const buffer_rsrc xrs = make_rsrc(L.x, (uint32_t)(((int64_t)(M - 1) * ldx + K) * 2));
        const buffer_rsrc srs = make_rsrc(L.s, (uint32_t)K * 4u);
#pragma unroll
        for (int u = 0; u < kUP; ++u) {
          if (u < up) {
            const int q = ht + u * kHT;
            const bool ok = q < units;
            sv[u][0] = load16(srs, ok ? q * 32 : kOutOfRange);
            sv[u][1] = load16(srs, ok ? q * 32 + 16 : kOutOfRange);
#pragma unroll
            for (int m = 0; m < MT; ++m)
              xv[u][m] = load16<kCoherent>(xrs, ok ? (int)((m * ldx + q * 8) * 2) : kOutOfRange);
          } else {
            sv[u][0] = sv[u][1] = (v4i){0, 0, 0, 0};
#pragma unroll
            for (int m = 0; m < MT; ++m) xv[u][m] = (v4i){0, 0, 0, 0};
          }
        }
      }
      if (!started) {
        __syncthreads();  // (1)
        started = true;
      }
      auto piece = [&](int u, int m, float v[8]) {
        const float sf[8] = {__int_as_float(sv[u][0].x), __int_as_float(sv[u][0].y),
                             __int_as_float(sv[u][0].z), __int_as_float(sv[u][0].w),
                             __int_as_float(sv[u][1].x), __int_as_float(sv[u][1].y),
                             __int_as_float(sv[u][1].z), __int_as_float(sv[u][1].w)};
        const uint32_t w4[4] = {(uint32_t)xv[u][m].x, (uint32_t)xv[u][m].y,
                                (uint32_t)xv[u][m].z, (uint32_t)xv[u][m].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t bits = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
          v[e] = bf16_to_f32(bits) * sf[e];  // xs = RN32(x * s)
        }
      };
      {
        float amax[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) amax[m] = 0.0f;
#pragma unroll
        for (int u = 0; u < kUP; ++u) {
          if (u < up) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              float v[8];
              piece(u, m, v);
#pragma unroll
              for (int e = 0; e < 8; ++e) amax[m] = fmaxf(amax[m], fabsf(v[e]));
            }
          }
        }
        // opaque copies: the products above must not stay live until the quantizer
#pragma unroll
        for (int u = 0; u < kUP; ++u) {
          asm volatile("" : "+v"(sv[u][0]), "+v"(sv[u][1]));
#pragma unroll
          for (int m = 0; m < MT; ++m) asm volatile("" : "+v"(xv[u][m]));
        }
        float wmax[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) wmax[m] = wave_max_nonneg(amax[m]);
        if (lane == 0) {
#pragma unroll
          for (int m = 0; m < MT; ++m) amax_part[hwave * 8 + m] = wmax[m];
          __hip_atomic_fetch_add(cnt, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
        }
      }
      lds_wait_at_least(cnt, kNH * (qseq + 1), wc);
      ++qseq;
      float row_amax = 0.0f;
      if (lane < MT) {
#pragma unroll
        for (int w = 0; w < kNH; ++w) row_amax = fmaxf(row_amax, amax_part[w * 8 + lane]);
      }
      const QParams lp = row_qparams(row_amax);
      if (hwave == 0 && lane < MT) qp[lane] = lp.scale;  // read back by this wavefront's epilogue
      float inv_row[MT];
#pragma unroll
      for (int m = 0; m < MT; ++m)
        inv_row[m] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lp.inv), m));
#pragma unroll
      for (int u = 0; u < kUP; ++u) {
        const int q = ht + u * kHT;
        if (u < up && q < units) {
#pragma unroll
          for (int m = 0; m < MT; ++m) {
            float v[8];
            piece(u, m, v);
            uint32_t cb[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) cb[e] = quant_code_biased(v[e], inv_row[m]);
            uint2 pk;
            pk.x = pack4_low_bytes(cb[0], cb[1], cb[2], cb[3]);
            pk.y = pack4_low_bytes(cb[4], cb[5], cb[6], cb[7]);
            *reinterpret_cast<uint2*>(codes + m * Ks + q * 8) = pk;
          }
        }
        // step u (K positions [u * 4096, (u + 1) * 4096)) of this wavefront is in LDS
        if (lane == 0)
          __hip_atomic_fetch_add(ready + u, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
      if (lane == 0)  // the fourth counter is kept in step with the others
        __hip_atomic_fetch_add(ready + 3, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }

    // ---- tiles: dequant epilogue
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
    uint16_t* y = L.y;
    int32_t* acc_out = L.acc_out;
    for (int t = 0; t < T; ++t) {
      const int tile = first + t;
      const int buf = tcount & 1;
      ++tcount;
      __syncthreads();  // partials of the tile published
      if (ht < 64) {
        const int tt = ht & 15;
        const int n0 = tile * 16 + 4 * (ht >> 4);
        if (tt < M) {
          v4i tot = {0, 0, 0, 0};
#pragma unroll
          for (int w = 0; w < kS; ++w)
            tot += *reinterpret_cast<const v4i*>(red + (buf * kS + w) * 256 + ht * 4);
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
          int oc = n0;
          bool has = true;
          if (swiglu) {
            // gated order: channels 0..7 of the tile are the gate and 8..15 the
            // up projections of outputs 8 tile .. + 7; the up values of this
            // thread's 4 outputs sit 32 lanes on
            uint32_t upv[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) upv[i] = (uint32_t)__shfl_xor((int)o[i], 32, kWave);
            has = (ht >> 4) < 2;
            oc = tile * 8 + 4 * (ht >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const float gv = bf16_to_f32(o[i]), uv = bf16_to_f32(upv[i]);
              const float sg = gv / (1.0f + expf(-gv));
              o[i] = f32_to_bf16_rne(sg * uv);
            }
          }
          if (has) {
            // agent-scope stores: the next link's workgroups read them in this launch
            __hip_atomic_store(
                reinterpret_cast<uint64_t*>(y + (size_t)tt * (swiglu ? N / 2 : N) + oc),
                (uint64_t)(o[0] | (o[1] << 16)) | ((uint64_t)(o[2] | (o[3] << 16)) << 32),
                __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (acc_out)
#pragma unroll
              for (int i = 0; i < 4; ++i) acc_out[(size_t)tt * N + n0 + i] = tv[i];
            if (lm_partials)
#pragma unroll
              for (int i = 0; i < 4; ++i) track(bf16_to_f32(o[i]), n0 + i);
          }
        }
      }
    }
    if (lm_partials && ht < 64) {
      // the four threads of token tt are lanes tt, tt + 16, tt + 32, tt + 48
#pragma unroll
      for (int off = 16; off <= 32; off <<= 1) {
        const float ov = __shfl_xor(am_v, off, kWave);
        const int oi = __shfl_xor(am_i, off, kWave);
        const float os = __shfl_xor(am_s, off, kWave);
        const float mx = fmaxf(am_v, ov);
        if (ap.psum) am_s = am_s * expf((am_v - mx) * ap.inv_t) + os * expf((ov - mx) * ap.inv_t);
        if (ov > am_v || (ov == am_v && oi < am_i)) am_i = oi;
        am_v = mx;
      }
      if (ht < M) {
        const size_t slot = (size_t)ht * G + b;
        ap.pmax[slot] = am_v;
        ap.pidx[slot] = am_i;
        if (ap.psum) ap.psum[slot] = am_s;
      }
    }
    // this workgroup's part of link li is stored: raise its progress word
    // (after the stores have completed when the next link reads them)
    if (hwave == 0) {
      if (consumed && T > 0) wait_stores_complete();
      if (lane == 0) store_flag(flag_word(progress, 0, b), base + (uint32_t)li + 1u);
    }
  }
  if (!started) __syncthreads();  // (1): no link had tiles here
  // a streamer wait gives up only before a tile barrier, all of which are behind
  if (ht == 0 && __hip_atomic_load(expired, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP))
    note_expired(wc, kWaitLds);
}

template <int MT, int NBUF>
__global__ __launch_bounds__(kThreads) void w8a8_chain_kernel(const quasar_chain_link* __restrict__ links,
                                                              int n, int M, int Kmax,
                                                              uint32_t* progress,
                                                              AcceptPartials ap, WaitCtl wc) {
  extern __shared__ __align__(16) char smem[];
  const Smem L = chain_smem(Kmax, MT);
  int8_t* codes = reinterpret_cast<int8_t*>(smem + L.codes);
  int32_t* red = reinterpret_cast<int32_t*>(smem + L.red);
  float* wsl = reinterpret_cast<float*>(smem + L.wsl);
  float* amax_part = reinterpret_cast<float*>(smem + L.amax);
  float* qp = reinterpret_cast<float*>(smem + L.qp);
  int* cnt = reinterpret_cast<int*>(smem + L.cnt);
  int* ready = reinterpret_cast<int*>(smem + L.ready);
  int* gate = reinterpret_cast<int*>(smem + L.gate);
  int* expired = reinterpret_cast<int*>(smem + L.expired);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid < 8) {  // ordered before use by barrier (1)
    if (tid == 0) *cnt = 0;
    if (tid == 1) *gate = 0;
    if (tid == 2) *expired = 0;
    if (tid < 4) ready[tid] = 0;
  }
  const int G = gridDim.x, b = blockIdx.x;
  if (wave < kS) {
    chain_streamer<MT, NBUF>(links, n, b, G, wave, lane, codes, red, wsl, ready, expired, wc);
  } else {
    chain_helper<MT>(links, n, M, b, G, tid - 64 * kS, wave - kS, lane, codes, red, wsl,
                     amax_part, qp, cnt, ready, gate, expired, progress, ap, wc);
  }
}

constexpr int kNBUF = 3;  // weight units in flight per streamer: 24 KB, 96 KB per compute unit

template <int MT>
hipError_t launch_chain_mt(const quasar_chain_link* links_dev, int n, int M, int Kmax, int G,
                           uint32_t* progress, const AcceptPartials& ap, const WaitCtl& wc,
                           hipStream_t st) {
  auto kernel = &w8a8_chain_kernel<MT, kNBUF>;
  static const hipError_t attr =
      hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                          hipFuncAttributeMaxDynamicSharedMemorySize,
                          chain_smem(kChainMaxK, MT).bytes);
  if (attr != hipSuccess) return attr;
  kernel<<<dim3(G), dim3(kThreads), chain_smem(Kmax, MT).bytes, st>>>(links_dev, n, M, Kmax,
                                                                       progress, ap, wc);
  return hipGetLastError();
}

}  // namespace

int chain_lds_bytes(int M, int Kmax) {
  const int mt = M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 6 ? 6 : 8));
  return chain_smem(Kmax, mt).bytes;
}

const char* chain_kernel_name(int M) {
  static const char* const names[4] = {
      "w8a8_chain_kernel<2, 3>", "w8a8_chain_kernel<4, 3>", "w8a8_chain_kernel<6, 3>",
      "w8a8_chain_kernel<8, 3>"};
  const int mt = M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 6 ? 6 : 8));
  return names[mt / 2 - 1];
}

hipError_t launch_chain(const quasar_chain_link* links_dev, int n, int M, int Kmax, int G,
                        void* workspace, const AcceptPartials* partials, hipStream_t st) {
  const WaitCtl wc = wait_ctl_for_current_device();
  if (!wc.status) return hipErrorInvalidSymbol;
  const AcceptPartials ap = partials ? *partials : AcceptPartials{nullptr, nullptr, nullptr, 0.0f};
  uint32_t* progress = static_cast<uint32_t*>(workspace);
  const int mt = M <= 2 ? 2 : (M <= 4 ? 4 : (M <= 6 ? 6 : 8));
  switch (mt) {
    case 2: return launch_chain_mt<2>(links_dev, n, M, Kmax, G, progress, ap, wc, st);
    case 4: return launch_chain_mt<4>(links_dev, n, M, Kmax, G, progress, ap, wc, st);
    case 6: return launch_chain_mt<6>(links_dev, n, M, Kmax, G, progress, ap, wc, st);
    default: return launch_chain_mt<8>(links_dev, n, M, Kmax, G, progress, ap, wc, st);
  }
}

}  // namespace quasar
