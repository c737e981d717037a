// One-launch W8A8 SmoothQuant linear for wide verify windows (9..128 tokens,
// or any window with K > 12288): online smoothing and dynamic per-token INT8
// quantization of the BF16 activations, the INT8 x INT8 -> INT32 product on
// the matrix cores against the resident INT8 weights, and BF16 dequantization
// [Quasar, pt page §2 execution pipeline items 2-4; zh page §2 items 2-3].
//
// A wide window is too large for the one-launch kernel of small windows,
// which keeps the whole quantized activation matrix in every compute unit's
// LDS (96 tokens x 4096 K positions is 384 KB; LDS is 160 KB).  Here the
// quantized activations go to global memory once and are streamed through a
// small LDS area next to the weights:
//
//   1. Rows.  Workgroup m < M smooths and quantizes token row m
//      (xs = RN32(x * s), absmax, scale, codes) into the workspace, then
//      publishes a per-workgroup flag.  The codes are stored fragment-major:
//      the 16 x 64 fragment of token block tb at K chunk c is one contiguous
//      1 KB at (tb * nch + c) KB, lane l = 16 g + r holding the 16 codes of
//      token 16 tb + r at K positions 64 c + 16 g .. + 15 (the MFMA B operand
//      order), so a fragment load is one contiguous 1 KB read.  Measured on
//      MI355X with every compute unit reading the same L2-resident 384 KB:
//      128 GB/s per compute unit this way, 37 GB/s with the 16 rows of a
//      fragment K bytes apart (row-major codes).  Every workgroup waits until the M row
//      flags are set -- a one-way grid barrier.  Meanwhile its streamer
//      wavefronts already have their first weights in flight.
//   2. Items.  The output channels are cut into groups of TG tiles of 16
//      channels (TG = 1, 2, 4 or 6: wide_tiles_per_group) and K into items of
//      256 positions (4 chunks of 64, one per streamer wavefront).  The
//      (group, item) sequence, group major, is divided into G equal
//      contiguous ranges, one per workgroup (stream-K): every workgroup
//      streams the same number of weight bytes whatever N and K are.  G is
//      the number of groups where they fit the device and K <= 8192 (each
//      workgroup owns one whole group), else one workgroup per compute unit.
//      With the token-block split (wide_token_split: groups of 2 or 3 tiles
//      from 64 tokens), each range is run by two workgroups of one XCD, each
//      on half of the token blocks.
//   3. Per item, each of the 4 streamer wavefronts loads one 1 KB chunk of
//      each of the group's TG tiles into registers and, right behind them, the
//      activation codes of that K chunk -- one 16 x 64 fragment per 16-token
//      block -- with direct-to-LDS buffer loads into a slot of its own, then
//      multiplies each fragment against the TG tiles.  Weights and codes of
//      NBUF items are in flight per wavefront.  A compute unit holds only a
//      bounded number of outstanding vector-memory requests and later
//      requests wait at issue, so codes loaded by a separate wavefront would
//      queue behind the weight stream and starve it; issued by the streamer
//      right behind its weights, they land with them and one in-order wait
//      count covers both.
//   4. At the end of a group (or of the range) the streamers hand their
//      partial sums to the four helper wavefronts, one tile at a time through a
//      double-buffered LDS area.  The epilogue sums the 4 partials (exact
//      INT32) and either dequantizes to BF16, or -- for a group whose first
//      item belongs to another workgroup -- stores the INT32 partial to the
//      workspace and raises a flag.  The workgroup that owns a group's first
//      item finishes that group, adding the partials of the workgroups that
//      own its later items.
//
// Synchronisation inside a workgroup uses monotonic LDS counters (no
// workgroup barrier after the first), so a stalled role never stalls
// another.  The streamers touch LDS only through inline assembly: the
// compiler cannot tell their LDS words from the slots the direct-to-LDS loads
// write and would otherwise wait for every load in flight before each access,
// while LDS executes a wavefront's accesses in issue order anyway.
//
// Across workgroups it uses the flag header of the caller's workspace (the
// protocol of quasar_sync.hpp): row flags (word b: workgroup b's token row is
// in the workspace) and partial flags (word 256 + b: its partial sum of a
// shared group is).  Workgroup b reads its row flag e at the start and raises
// it to e + 1 once per launch, so a flag equal to e + 1 marks this launch's
// data; the header must hold equal words (zeros) before the workspace's first
// use and is never reset (a launch raises the row-flag words beyond its grid
// as well, so launches of different grids can share a workspace).  The grid
// is at most one workgroup per compute unit and all of them must be resident
// at once; every wait is bounded, and one that gives
// up sets a bit of the device status word (undefined outputs) instead of
// hanging.
#include <mutex>
#include <string>
#include <vector>

#include "quasar_device.hpp"
#include "quasar_internal.hpp"
#include "quasar_sync.hpp"

namespace quasar {
namespace {

constexpr int kS = 4;        // streamer wavefronts (one 64-wide K chunk each per item)
constexpr int kMaxTG = 4;    // 16-channel tiles per group: 1, 2 or 4 ...
constexpr int kWideTG = 6;   // ... or 6 (beyond 4 tiles per CU at 48 to 96 tokens)
constexpr int kHelpers = 4;  // row quantizer, then epilogue wavefronts
constexpr int kThreads = 64 * (kS + kHelpers);
constexpr int kRowPieces = 8;  // 8-element pieces per helper thread kept in registers

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt at their
// maxima so they are not waited for).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8); }
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Items in flight per streamer (NBUF) for MB 16-token blocks, TG tiles per
// group and F code fragments per token block and item (1 for INT8 weights, 2
// for 4-bit weights, whose 1 KB weight block holds two 64-wide K chunks): the
// code slots (4 streamers x NBUF items x F MB KB) and the partial-sum area
// (2 x 4 x MB KB) stay within 150 KB of LDS, and the loads in flight per
// wavefront ((NBUF - 1) items of TG + F MB, plus one item's F MB code loads)
// within what the 6-bit vmcnt counter can wait for.  4 items with INT8
// weights and 2 with 4-bit ones (whose items carry twice the code fragments):
// measured against 8 items, QKV, O and down at 96 tokens 16.0, 13.3, 25.6 ->
// 15.0, 12.6, 24.9 us, at 48 tokens 13.3, 11.6, 20.2 -> 13.1, 11.3, 19.8, and
// with 4-bit weights at 96 tokens 13.8, 12.0 -> 12.4, 11.2 (2 or 3 items
// were slower with INT8 weights, 6 in between).  Groups of 6 tiles keep 2
// items in flight: their 6 x MB accumulators leave no registers for more (3
// or 4, where they fit, measured ~1 us slower on gate_up).
constexpr int wide_nbuf(int MB, int TG, int F = 1) {
  int nb = TG > kMaxTG || F == 2 ? 2 : 4;
  while (nb > 2 && (kS * nb * F * MB + 2 * kS * MB > 150 || (nb - 1) * (TG + F * MB) + F * MB > 63))
    --nb;
  return nb;
}
template <int MB, int TG, int F = 1>
struct Wide {
  static constexpr int NBUF = wide_nbuf(MB, TG, F);
  static constexpr int SLOTS = kS * NBUF * F * MB * 1024;
  static constexpr int RED = 2 * kS * MB * 1024;
  static constexpr int SYNC = 256;
  static constexpr int LDS = SLOTS + RED + SYNC;
};
template <int MB, int F>
constexpr bool wide_fits() {
  return Wide<MB, 1, F>::LDS <= 150 * 1024 && Wide<MB, 2, F>::LDS <= 150 * 1024 &&
         Wide<MB, 4, F>::LDS <= 150 * 1024 &&
         (Wide<MB, 1, F>::NBUF - 1) * (1 + F * MB) + F * MB <= 63 &&
         (Wide<MB, 2, F>::NBUF - 1) * (2 + F * MB) + F * MB <= 63 &&
         (Wide<MB, 4, F>::NBUF - 1) * (4 + F * MB) + F * MB <= 63;
}
// 4-bit weights: up to 6 token blocks (96 tokens)
constexpr int kWideMaxMbW4 = 6;
static_assert(wide_fits<1, 1>() && wide_fits<2, 1>() && wide_fits<3, 1>() && wide_fits<4, 1>() &&
                  wide_fits<5, 1>() && wide_fits<6, 1>() && wide_fits<7, 1>() &&
                  wide_fits<8, 1>() && wide_fits<1, 2>() && wide_fits<2, 2>() &&
                  wide_fits<3, 2>() && wide_fits<4, 2>() && wide_fits<5, 2>() && wide_fits<6, 2>(),
              "LDS budget, and in-flight loads within the 6-bit vmcnt");
// groups of 6 tiles: 1 to 6 token blocks
template <int MB, int F>
constexpr bool wide_fits_tg6() {
  return Wide<MB, kWideTG, F>::LDS <= 150 * 1024 &&
         (Wide<MB, kWideTG, F>::NBUF - 1) * (kWideTG + F * MB) + F * MB <= 63;
}
static_assert(wide_fits_tg6<2, 1>() && wide_fits_tg6<1, 2>() && wide_fits_tg6<2, 2>() &&
                  wide_fits_tg6<3, 1>() && wide_fits_tg6<4, 1>() && wide_fits_tg6<5, 1>() &&
                  wide_fits_tg6<6, 1>() && wide_fits_tg6<3, 2>() && wide_fits_tg6<4, 2>() &&
                  wide_fits_tg6<5, 2>() && wide_fits_tg6<6, 2>(),
              "groups of 6 tiles: LDS budget and in-flight loads");

// LDS synchronisation words (int indices into the SYNC area)
enum : int {
  kRedReady = 16,  // [2] per parity: streamers that published a tile round
  kRedFree = 18,   // [2] per parity: epilogue wavefronts that consumed a round
  kRowDone = 20,   // helper wavefronts whose row codes are stored
  kAmaxCnt = 21,   // helper wavefronts that published their row maximum
  kGate = 22,      // 1 once every token row of the launch is in the workspace
  kPartDone = 23,  // epilogue wavefronts whose partial sums are stored
  kAmax = 24,      // float [4] per-helper row maxima
  kFlagOut = 28,   // 1 once this workgroup's row flag store has been issued
  kSyncWords = 32
};

// LDS accesses of the streamer wavefronts (see the note above), by LDS byte
// address.
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)p);
}

__device__ __forceinline__ int lds_read_asm(uint32_t addr) {
  int v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

__device__ __forceinline__ void lds_add_asm(uint32_t addr, int v) {
  asm volatile("ds_add_u32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ v4i lds_read16_asm(uint32_t addr) {  // no wait: see lds_wait_reads
  v4i v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr) : "memory");
  return v;
}

__device__ __forceinline__ void lds_write16_asm(uint32_t addr, v4i v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ void lds_wait_reads() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// Bounded wait until an LDS counter reaches `target`, for the streamers.  On
// expiry the status word is set with a global atomic: it counts as one more
// outstanding vector-memory operation, which only makes the streamers' exact
// waits below wait for one more load.
__device__ __forceinline__ void lds_wait_ge_asm(uint32_t addr, int target, const WaitCtl& wc) {
  const int t = target + (int)wc.bias;
  for (int spin = 0;; ++spin) {
    if (lds_read_asm(addr) >= t) break;
    if (spin >= wc.spin_lds) {
      note_expired(wc, kWaitLds);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}

__device__ __forceinline__ int lds_load(const int* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

__device__ __forceinline__ void lds_add(int* p, int v) {
  __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Stores another workgroup reads during the same launch: agent-scope
// (write-through) stores, ordered before the flag that publishes them by a
// release fence (quasar_sync.hpp).
__device__ __forceinline__ void store8_device(void* p, uint2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p),
                     (uint64_t)v.x | ((uint64_t)v.y << 32), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store16_device(int32_t* p, v4i v) {
  store8_device(p, make_uint2((uint32_t)v.x, (uint32_t)v.y));
  store8_device(p + 2, make_uint2((uint32_t)v.z, (uint32_t)v.w));
}

// Wait until every store this wavefront issued has completed, i.e. is visible
// device-wide for the device-scope stores above; flags are raised after it.
__device__ __forceinline__ void wait_stores_done() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  asm volatile("" ::: "memory");
}


// Item ranges: the (group, item) sequence of U items is split into G equal
// contiguous ranges.
__host__ __device__ inline int range_start(int b, int U, int G) {
  return (int)((int64_t)b * U / G);
}

// Token-block split: the workgroup that runs range c on half `mpart` of the
// token blocks.  Workgroup b runs on XCD b % 8, so the two workgroups of a
// range, b and b + 8, share an XCD and read the range's weights through its L2.
__host__ __device__ inline int wide_split_wg(int c, int mpart) {
  return (c & 7) | (mpart << 3) | ((c >> 3) << 4);
}

// ---------------------------------------------------------------------------
// Streamer role: weights and codes -> MFMA -> per-tile partial rounds.
// WB = 8: a weight block is one 64-wide K chunk of a tile (the INT8 layout);
// WB = 4: it is the pair of chunks 2c, 2c + 1 of the 4-bit layout, so an item
// spans 512 K positions and each block meets the codes of two chunks (F = 2).
// SPLIT: the workgroup multiplies token blocks tb0 .. tb0 + MB - 1 of the 2 MB
// blocks of the code matrix (otherwise blocks 0 .. MB - 1 of MB).
// ---------------------------------------------------------------------------
template <int MB, int TG, int WB, bool SPLIT>
__device__ __forceinline__ void wide_streamer(const int8_t* __restrict__ wq,
                                              const int8_t* __restrict__ qx, int M, int K,
                                              int tiles, int nch, int P, int i0, int n, int w,
                                              int lane, bool quantizer, int tb0_split,
                                              char* slots,
                                              int32_t* red, int* sync, const WaitCtl& wc) {
  constexpr int F = WB == 4 ? 2 : 1;
  using C = Wide<MB, TG, F>;
  constexpr int NB = C::NBUF;
  const int voff = lane * 16;
  const int nwc = WB == 4 ? K >> 7 : nch;  // weight blocks per tile

  // Weights of the next item into register buffer bb: block (item * 4 + w) of
  // the group's tiles, 1 KB each, zeros past the range, N or K.
  v4i a[NB][TG];
  int ig = i0 / P, ip = i0 - (i0 / P) * P, wissued = 0;
  auto issue_weights = [&](int bb) {
    const bool live = wissued < n;
    const int c = ip * kS + w;
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      const int t = ig * TG + tt;
      const bool ok = live && t < tiles && c < nwc;
      const buffer_rsrc rs =
          make_rsrc(wq + ((size_t)(ok ? t : 0) * nwc + (ok ? c : 0)) * 1024, ok ? 1024u : 0u);
      a[bb][tt] = load16<kNonTemporal>(rs, voff);
    }
    ++wissued;
    if (++ip == P) {
      ip = 0;
      ++ig;
    }
  };
  // Codes of the next item into this streamer's LDS slot bb: fragment (f, tb)
  // holds token block tb0 + tb (of the MBT blocks of the code matrix) at K
  // chunk F (item * 4 + w) + f, one contiguous 1 KB
  // of the fragment-major codes, which the direct-to-LDS load stores in lane
  // order.  Token rows >= M hold whatever the workspace held: they only reach
  // output rows that are never stored.  A chunk past K meets zero weights.
  constexpr int MBT = SPLIT ? 2 * MB : MB;
  const int tb0 = SPLIT ? tb0_split : 0;
  const buffer_rsrc qrs = make_rsrc(qx, (uint32_t)MBT * (uint32_t)nch * 1024u);
  const int lane_off = lane * 16;
  char* my_slots = slots + w * NB * F * MB * 1024;
  int cp_issue = i0 - (i0 / P) * P, cissued = 0;
  auto issue_codes = [&](int bb) {
    const bool live = cissued < n;
    const int c = cp_issue * kS + w;
#pragma unroll
    for (int f = 0; f < F; ++f)
#pragma unroll
      for (int tb = 0; tb < MB; ++tb)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            qrs, (__attribute__((address_space(3))) void*)(my_slots + ((bb * F + f) * MB + tb) * 1024),
            16, live ? lane_off + ((tb0 + tb) * nch + F * c + f) * 1024 : kOutOfRange, 0, 0,
            kCoherent);
    ++cissued;
    if (++cp_issue == P) cp_issue = 0;
  };

  __syncthreads();  // (1) the row quantizer's activation loads are queued first
  if (n == 0) return;
  // A compute unit serves its vector-memory requests in order, and the row
  // quantizer's code stores, its flag and every flag poll sit on the critical
  // path of the launch: in a workgroup that quantizes a row, the weight stream
  // starts once the row is out, so those stores do not queue behind it.  (The
  // other workgroups' first weights have landed by the time the flags are
  // polled.)
  if (quantizer) lds_wait_ge_asm(lds_address(sync + kFlagOut), 1, wc);
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) issue_weights(bb);
  // the codes exist once every token row of the launch is in the workspace
  lds_wait_ge_asm(lds_address(sync + kGate), 1, wc);
#pragma unroll
  for (int bb = 0; bb < NB; ++bb) issue_codes(bb);
  __builtin_amdgcn_sched_barrier(0);  // keep the loop below from rotating into the issues

  v4i acc[TG][MB];
#pragma unroll
  for (int tt = 0; tt < TG; ++tt)
#pragma unroll
    for (int tb = 0; tb < MB; ++tb) acc[tt][tb] = (v4i){0, 0, 0, 0};

  const uint32_t slot_addr = lds_address(my_slots) + lane * 16;
  const uint32_t red_addr = lds_address(red) + w * MB * 1024 + lane * 16;
  int cp = i0 - (i0 / P) * P;  // consume pointer: item within its group
  int round = 0;
  for (int jb = 0; jb < n; jb += NB) {
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) {
      const int j = jb + bb;
      if (j < n) {
        // Item j's weights and codes have landed once at most the loads issued
        // after its codes are outstanding (loads complete in issue order):
        // (NB - 1) F MB code loads of later items, plus the weights of the
        // items issued since -- (NB - 1) F MB + min(j, NB - 1) TG in all.
        switch (j < NB - 1 ? j : NB - 1) {
          case 0: __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * F * MB)); break;
          case 1: __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * F * MB + 1 * TG)); break;
          case 2: __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * F * MB + 2 * TG)); break;
          case 3: __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * F * MB + 3 * TG)); break;
          case 4: __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * F * MB + 4 * TG)); break;
          case 5: __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * F * MB + 5 * TG)); break;
          case 6: __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * F * MB + 6 * TG)); break;
          default: __builtin_amdgcn_s_waitcnt(vmcnt_imm((NB - 1) * F * MB + 7 * TG)); break;
        }
        if constexpr (WB == 4 && TG > kMaxTG) {
          // groups of 6 tiles with 4-bit weights: chunk 2c's codes first, then
          // chunk 2c + 1's, so only half of the item's code fragments are in
          // registers at a time
          const v4u hm = {0xF0F0F0F0u, 0xF0F0F0F0u, 0xF0F0F0F0u, 0xF0F0F0F0u};
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            v4i bq[MB];
#pragma unroll
            for (int tb = 0; tb < MB; ++tb)
              bq[tb] = lds_read16_asm(slot_addr + ((bb * F + f) * MB + tb) * 1024);
            lds_wait_reads();
#pragma unroll
            for (int tb = 0; tb < MB; ++tb) asm volatile("" : "+v"(bq[tb]));
#pragma unroll
            for (int tt = 0; tt < TG; ++tt) {
              const v4u v = __builtin_bit_cast(v4u, a[bb][tt]);
              const v4i q = __builtin_bit_cast(v4i, f == 0 ? ((v << 4u) & hm) : (v & hm));
#pragma unroll
              for (int tb = 0; tb < MB; ++tb) acc[tt][tb] = mfma_i8_16x16x64(q, bq[tb], acc[tt][tb]);
            }
          }
        } else {
        v4i bf[F * MB];
#pragma unroll
        for (int i = 0; i < F * MB; ++i)
          bf[i] = lds_read16_asm(slot_addr + (bb * F * MB + i) * 1024);
        lds_wait_reads();
#pragma unroll
        for (int i = 0; i < F * MB; ++i) asm volatile("" : "+v"(bf[i]));
#pragma unroll
        for (int tt = 0; tt < TG; ++tt) {
          if constexpr (WB == 4) {
            // each byte's low nibble is chunk 2c's code, its high nibble chunk
            // 2c + 1's: both times 16 as exact int8 values (the epilogue
            // divides the sums by 16)
            const v4u v = __builtin_bit_cast(v4u, a[bb][tt]);
            const v4u hm = {0xF0F0F0F0u, 0xF0F0F0F0u, 0xF0F0F0F0u, 0xF0F0F0F0u};
            const v4i lo = __builtin_bit_cast(v4i, (v << 4u) & hm);
            const v4i hi = __builtin_bit_cast(v4i, v & hm);
#pragma unroll
            for (int tb = 0; tb < MB; ++tb) {
              acc[tt][tb] = mfma_i8_16x16x64(lo, bf[tb], acc[tt][tb]);
              acc[tt][tb] = mfma_i8_16x16x64(hi, bf[MB + tb], acc[tt][tb]);
            }
          } else {
#pragma unroll
            for (int tb = 0; tb < MB; ++tb)
              acc[tt][tb] = mfma_i8_16x16x64(a[bb][tt], bf[tb], acc[tt][tb]);
          }
        }
        }
      }
      // item j + NB into buffer bb and slot bb (slot bb's codes are in
      // registers now), or zeros past the range
      issue_weights(bb);
      issue_codes(bb);
      if (j < n) {
        const bool group_end = cp == P - 1 || j == n - 1;
        if (group_end) {
#pragma unroll
          for (int tt = 0; tt < TG; ++tt) {
            const int par = round & 1;
            if (round >= 2)
              lds_wait_ge_asm(lds_address(sync + kRedFree + par), kHelpers * (round >> 1), wc);
#pragma unroll
            for (int tb = 0; tb < MB; ++tb) {
              lds_write16_asm(red_addr + (par * kS * MB + tb) * 1024, acc[tt][tb]);
              acc[tt][tb] = (v4i){0, 0, 0, 0};
            }
            if (lane == 0) lds_add_asm(lds_address(sync + kRedReady + par), 1);
            ++round;
          }
        }
        if (++cp == P) cp = 0;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Helper prologue: smooth and quantize token row `m` into the workspace.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void quantize_row_compute(const uint16_t* __restrict__ x,
                                                     const float* __restrict__ s, int m, int K,
                                                     int ht, int hw, int lane, const v4i (&xv)[kRowPieces],
                                                     const v4i (&sv)[kRowPieces][2], bool in_regs,
                                                     int8_t* __restrict__ qx, float* __restrict__ sx,
                                                     int* sync, const WaitCtl& wc) {
  const int units = K >> 3;
  const buffer_rsrc xrs = make_rsrc(x + (size_t)m * K, (uint32_t)K * 2u);
  const buffer_rsrc srs = make_rsrc(s, (uint32_t)K * 4u);
  auto piece = [&](const v4i& xq, const v4i& s0, const v4i& s1, float v[8]) {
    const float sf[8] = {__int_as_float(s0.x), __int_as_float(s0.y), __int_as_float(s0.z),
                         __int_as_float(s0.w), __int_as_float(s1.x), __int_as_float(s1.y),
                         __int_as_float(s1.z), __int_as_float(s1.w)};
    const uint32_t w4[4] = {(uint32_t)xq.x, (uint32_t)xq.y, (uint32_t)xq.z, (uint32_t)xq.w};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t bits = (e & 1) ? (w4[e >> 1] >> 16) : (w4[e >> 1] & 0xffffu);
      v[e] = bf16_to_f32(bits) * sf[e];  // xs = RN32(x * s)
    }
  };
  // absmax of the row (pieces past K read as zero)
  float amax = 0.0f;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kRowPieces; ++u) {
      float v[8];
      piece(xv[u], sv[u][0], sv[u][1], v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
  } else {
    for (int q = ht; q < units; q += 64 * kHelpers) {
      float v[8];
      piece(load16(xrs, q * 16), load16(srs, q * 32), load16(srs, q * 32 + 16), v);
#pragma unroll
      for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
    }
  }
  const float wmax = wave_max_nonneg(amax);
  float* amax_part = reinterpret_cast<float*>(sync + kAmax);
  if (lane == 0) {
    amax_part[hw] = wmax;
    asm volatile("" ::: "memory");
    lds_add(sync + kAmaxCnt, 1);
  }
  lds_wait_at_least(sync + kAmaxCnt, kHelpers, wc);
  float row_amax = 0.0f;
#pragma unroll
  for (int h = 0; h < kHelpers; ++h) row_amax = fmaxf(row_amax, amax_part[h]);
  const QParams qp = row_qparams(row_amax);

  // piece q (K positions 8 q .. 8 q + 7) of token m: byte 8 (q % 2) of lane
  // 16 g + m % 16 of the fragment of token block m / 16 at K chunk q / 8,
  // g = (q / 2) % 4
  const int nch = (K + 63) >> 6;
  int8_t* qblk = qx + (size_t)(m >> 4) * nch * 1024 + (m & 15) * 16;
  auto emit = [&](int q, const float v[8]) {
    uint32_t cb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) cb[e] = quant_code_biased(v[e], qp.inv);
    uint2 pk;
    pk.x = pack4_low_bytes(cb[0], cb[1], cb[2], cb[3]);
    pk.y = pack4_low_bytes(cb[4], cb[5], cb[6], cb[7]);
    store8_device(qblk + (q >> 3) * 1024 + ((q >> 1) & 3) * 256 + (q & 1) * 8, pk);
  };
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kRowPieces; ++u) {
      const int q = ht + u * 64 * kHelpers;
      if (q < units) {
        float v[8];
        piece(xv[u], sv[u][0], sv[u][1], v);
        emit(q, v);
      }
    }
  } else {
    for (int q = ht; q < units; q += 64 * kHelpers) {
      float v[8];
      piece(load16(xrs, q * 16), load16(srs, q * 32), load16(srs, q * 32 + 16), v);
      emit(q, v);
    }
  }
  if (ht == 0)
    __hip_atomic_store(sx + m, qp.scale, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Helper prologue: quantize token row b (b < M) into the workspace and raise
// this workgroup's row flag, then wait until the token rows [mlo, mhi) this
// workgroup multiplies are there (helper wavefront 0 polls their flags with
// agent-scope loads; the rows are read only after this).  Contains the workgroup
// barrier (1).  Returns false when the workgroup has no items; `e` is this
// workgroup's row flag before the launch.
// ---------------------------------------------------------------------------
template <bool SPLIT>
__device__ __forceinline__ bool wide_rows_and_gate(const uint16_t* __restrict__ x,
                                                   const float* __restrict__ s, int M, int K, int b,
                                                   int G, int n, int mlo, int mhi, int ht,
                                                   int hw, int lane,
                                                   int8_t* __restrict__ qx, float* __restrict__ sx,
                                                   uint32_t* flags, int* sync, uint32_t& e,
                                                   const WaitCtl& wc) {
  e = load_flag(flag_word(flags, 0, b));
  const bool quantizer = b < M;
  const int units = K >> 3;
  const bool in_regs = units <= kRowPieces * 64 * kHelpers;
  v4i xv[kRowPieces], sv[kRowPieces][2];
  if (quantizer && in_regs) {
    const buffer_rsrc xrs = make_rsrc(x + (size_t)b * K, (uint32_t)K * 2u);
    const buffer_rsrc srs = make_rsrc(s, (uint32_t)K * 4u);
#pragma unroll
    for (int u = 0; u < kRowPieces; ++u) {
      const int q = ht + u * 64 * kHelpers;
      const bool ok = q < units;
      xv[u] = load16(xrs, ok ? q * 16 : kOutOfRange);
      sv[u][0] = load16(srs, ok ? q * 32 : kOutOfRange);
      sv[u][1] = load16(srs, ok ? q * 32 + 16 : kOutOfRange);
    }
  }
  __syncthreads();  // (1)

  // Row codes and scale go out with agent-scope stores; once every helper
  // wavefront's stores have completed, the row flag is raised behind a
  // release fence.
  if (quantizer) {
    quantize_row_compute(x, s, b, K, ht, hw, lane, xv, sv, in_regs, qx, sx, sync, wc);
    wait_stores_done();
    if (lane == 0) lds_add(sync + kRowDone, 1);
  }
  if (ht == 0) {
    if (quantizer) lds_wait_at_least(sync + kRowDone, kHelpers, wc);
    store_flag(flag_word(flags, 0, b), e + 1u);
    asm volatile("" ::: "memory");
    lds_add(sync + kFlagOut, 1);  // the flag is queued ahead of the weight stream
    // The slots beyond this launch's grid advance too (no launch reads them
    // before it ends), so that every slot's word keeps counting the launches
    // on this workspace whatever grid each of them had.
    for (int sl = b + G; sl < kFlagSlots; sl += G) store_flag(flag_word(flags, 0, sl), e + 1u);
  }
  if (n == 0) return false;

  if (hw == 0) {
    const uint32_t target = e + 1u + wc.bias;
    bool ok = false;
    for (int spin = 0;; ++spin) {
      bool ready = true;
      for (int m = (SPLIT ? mlo : 0) + lane; m < (SPLIT ? mhi : M); m += 64)
        ready &= load_flag(flag_word(flags, 0, m)) == target;
      if (__builtin_amdgcn_ballot_w64(!ready) == 0) {
        ok = true;
        break;
      }
      if (spin >= wc.spin_global) break;
      __builtin_amdgcn_s_sleep(1);
    }
    if (!ok && lane == 0) note_expired(wc, kWaitRows);
    after_poll();
    if (lane == 0) lds_add(sync + kGate, 1);
  } else {
    lds_wait_at_least(sync + kGate, 1, wc);
  }
  return true;
}

// ---------------------------------------------------------------------------
// Epilogue role.  Thread et (0..255) owns slots et + 256 k of a tile round:
// slot s = 64 tb + l is lane l of token block tb, i.e. token 16 (tb0 + tb) +
// l % 16 and the 4 channels 4 (l / 16) .. + 3 of the tile (the MFMA result
// layout).  Ranges are numbered r = 0..G-1 (G ranges); range c of this
// workgroup's half of the token blocks belongs to workgroup wg_of(c), whose
// number also indexes its partial-sum slot and partial flag.  No
// global load waits inside a round: the weight scales of a group are fetched
// while the streamers are still on it, and the partial sums of the workgroups
// that own the rest of a finalized group are summed once, before its rounds.
// ---------------------------------------------------------------------------
template <int MB, int TG, int WB, bool SPLIT>
__device__ __forceinline__ void wide_epilogue(const float* __restrict__ wscale,
                                              const float* __restrict__ sx, int M, int N, int P,
                                              int U, int G, int r, int bp, int tb0, int i0,
                                              int n, uint32_t e,
                                              int et, int lane, const int32_t* red, int* sync,
                                              int32_t* __restrict__ partials, uint32_t* flags,
                                              uint16_t* __restrict__ y,
                                              int32_t* __restrict__ acc_out, const WaitCtl& wc) {
  constexpr int KS = (MB + 3) / 4;           // slots per thread and round
  constexpr int kPartInts = (TG > kMaxTG ? TG : kMaxTG) * MB * 256;  // one workgroup's partial sums
  const int ln = et & 63;
  if (!SPLIT) tb0 = 0;
  const int mpart = (bp >> 3) & 1;
  auto wg_of = [&](int c) { return SPLIT ? wide_split_wg(c, mpart) : c; };
  float sxv[KS];
#pragma unroll
  for (int k = 0; k < KS; ++k) {
    const int tok = (tb0 + (et >> 6) + 4 * k) * 16 + (ln & 15);
    sxv[k] = tok < M ? load_coherent(sx + tok) : 0.0f;  // written by workgroup tok
  }
  const buffer_rsrc wrs = make_rsrc(wscale, (uint32_t)N * 4u);
  float ws[TG][4];  // weight scales of the group's 4 channels per tile of this thread
  auto fetch_ws = [&](int g) {
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        ws[tt][i] = __int_as_float(load4(wrs, (((g * TG + tt) * 16) + 4 * (ln >> 4) + i) * 4));
  };
  const int g_first = i0 / P, g_last = (i0 + n - 1) / P;
  fetch_ws(g_first);
  int round = 0;
  for (int g = g_first; g <= g_last; ++g) {
    const bool writer = g == g_first && i0 % P != 0;
    const bool finalizer = !writer && (i0 + n) < (g + 1) * P;
    v4i other[TG][KS];  // partial sums of the other owners of group g
#pragma unroll
    for (int tt = 0; tt < TG; ++tt)
#pragma unroll
      for (int k = 0; k < KS; ++k) other[tt][k] = (v4i){0, 0, 0, 0};
    if (finalizer && TG * KS > 8) {
      // groups of many tiles and token blocks: the contributors one after the
      // other (their partial sums fill the registers the streamers leave)
      for (int c = r + 1; c < G && range_start(c, U, G) < (g + 1) * P; ++c) {
        if (range_start(c + 1, U, G) == range_start(c, U, G)) continue;  // empty range
        const int cw = wg_of(c);
        for (int spin = 0;; ++spin) {
          if (load_flag(flag_word(flags, 1, cw)) == e + 1u + wc.bias) break;
          if (spin >= wc.spin_global) {
            if (lane == 0) note_expired(wc, kWaitPartials);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
        after_poll();  // the partial sums are read after the flag, agent-scope
        const buffer_rsrc prs =
            make_rsrc(partials + (size_t)cw * kPartInts, (uint32_t)kPartInts * 4u);
#pragma unroll
        for (int tt = 0; tt < TG; ++tt)
#pragma unroll
          for (int k = 0; k < KS; ++k) {
            const int sidx = et + 256 * k;
            if (sidx < MB * 64)
              other[tt][k] += load16<kCoherent>(prs, ((tt * MB + (sidx >> 6)) * 256 + ln * 4) * 4);
          }
      }
    } else if (finalizer) {
      // contributors: the non-empty ranges c_lo .. c_hi - 1 after r that start
      // inside group g (each owner wrote its partial sum of g first, then its
      // flag).  Lane j polls contributor c_lo + j, so all flags are waited for
      // together, and the partial sums are then loaded up to four contributors
      // at a time (as many as 32 registers hold): a group split over several
      // workgroups (a small N) pays one hand-off, not one per contributor.
      constexpr int kBatch = TG * KS <= 2 ? 4 : (TG * KS <= 4 ? 2 : 1);  // <= 32 registers
      // range c starts before item X = (g + 1) P exactly when c < X G / U
      const int c_lo = r + 1;
      const int c_hi =
          (int)min((int64_t)G, ((int64_t)(g + 1) * P * G + U - 1) / U);
      const uint32_t target = e + 1u + wc.bias;
      // one descriptor over every workgroup's partial-sum slot
      const buffer_rsrc prs =
          make_rsrc(partials, (uint32_t)kWideMaxGrid * (uint32_t)kPartInts * 4u);
      for (int c0 = c_lo; c0 < c_hi; c0 += 64) {
        const int nc = min(64, c_hi - c0);
        // an empty range writes no partial sums.  Ranges are empty only when
        // U < G (then (c + 1) U <= 256 * 256 fits 32 bits): range c is not
        // empty exactly when a multiple of G lies in (c U, (c + 1) U].
        const int c = c0 + lane;
        const bool mine = lane < nc && (U >= G || (unsigned)((c + 1) * U) % (unsigned)G <
                                                      (unsigned)U);
        const uint64_t live = __builtin_amdgcn_ballot_w64(mine);
        bool ok = false;
        for (int spin = 0;; ++spin) {
          const bool ready = !mine || load_flag(flag_word(flags, 1, wg_of(c))) == target;
          if (__builtin_amdgcn_ballot_w64(!ready) == 0) {
            ok = true;
            break;
          }
          if (spin >= wc.spin_global) break;
          __builtin_amdgcn_s_sleep(1);
        }
        if (!ok && lane == 0) note_expired(wc, kWaitPartials);
        after_poll();  // the partial sums are read after the flags, agent-scope
        for (int j0 = 0; j0 < nc; j0 += kBatch) {
          v4i part[kBatch][TG][KS];
#pragma unroll
          for (int j = 0; j < kBatch; ++j) {
            // an empty range or one past the group reads zeros
            const bool lv = j0 + j < nc && ((live >> (j0 + j)) & 1u);
            const int base = (lv ? wg_of(c0 + j0 + j) : 0) * kPartInts;
#pragma unroll
            for (int tt = 0; tt < TG; ++tt)
#pragma unroll
              for (int k = 0; k < KS; ++k) {
                const int sidx = et + 256 * k;
                part[j][tt][k] = load16<kCoherent>(
                    prs, lv && sidx < MB * 64
                             ? (base + (tt * MB + (sidx >> 6)) * 256 + ln * 4) * 4
                             : kOutOfRange);
              }
          }
#pragma unroll
          for (int j = 0; j < kBatch; ++j)
#pragma unroll
            for (int tt = 0; tt < TG; ++tt)
#pragma unroll
              for (int k = 0; k < KS; ++k) other[tt][k] += part[j][tt][k];
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < TG; ++tt) {
      const int par = round & 1;
      lds_wait_at_least(sync + kRedReady + par, kS * ((round >> 1) + 1), wc);
      const int n0 = (g * TG + tt) * 16 + 4 * (ln >> 4);
#pragma unroll
      for (int k = 0; k < KS; ++k) {
        const int sidx = et + 256 * k;
        if (sidx < MB * 64) {
          const int tb = sidx >> 6;
          v4i tot = other[tt][k];
#pragma unroll
          for (int w = 0; w < kS; ++w)
            tot += *reinterpret_cast<const v4i*>(red + ((par * kS + w) * MB + tb) * 256 + ln * 4);
          if (writer) {
            store16_device(partials + (size_t)bp * kPartInts + (tt * MB + tb) * 256 + ln * 4, tot);
          } else {
            const int tok = (tb0 + tb) * 16 + (ln & 15);
            if (tok < M && n0 < N) {
              // 4-bit weights: the sums are 16 times the products (exact shift)
              constexpr int sh = WB == 4 ? 4 : 0;
              const int tv[4] = {tot.x >> sh, tot.y >> sh, tot.z >> sh, tot.w >> sh};
              uint32_t o[4];
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                float v = (float)tv[i];  // round to nearest even
                v = v * sxv[k];
                v = v * ws[tt][i];
                o[i] = f32_to_bf16_rne(v);
              }
              uint16_t* yr = y + (size_t)tok * N;
              if (n0 + 3 < N && ((reinterpret_cast<uintptr_t>(yr + n0) & 7) == 0)) {
                uint2 pk;
                pk.x = o[0] | (o[1] << 16);
                pk.y = o[2] | (o[3] << 16);
                *reinterpret_cast<uint2*>(yr + n0) = pk;
              } else {
                for (int i = 0; i < 4 && n0 + i < N; ++i) yr[n0 + i] = (uint16_t)o[i];
              }
              if (acc_out)
                for (int i = 0; i < 4 && n0 + i < N; ++i) acc_out[(size_t)tok * N + n0 + i] = tv[i];
            }
          }
        }
      }
      asm volatile("" ::: "memory");  // the reads of this round precede the count
      if (lane == 0) lds_add(sync + kRedFree + par, 1);
      ++round;
    }
    if (g < g_last) fetch_ws(g + 1);  // lands while the streamers work on g + 1
    if (writer) {
      // both epilogue wavefronts' partial-sum stores complete, then one
      // raises this workgroup's partial flag
      wait_stores_done();
      if (lane == 0) lds_add(sync + kPartDone, 1);
      if (et == 0) {
        lds_wait_at_least(sync + kPartDone, kHelpers, wc);
        store_flag(flag_word(flags, 1, bp), e + 1u);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// The kernel: 4 streamer wavefronts, then 4 helper wavefronts (they quantize
// the workgroup's token row, then run the epilogue).  One body for INT8 (WB =
// 8) and 4-bit (WB = 4) weights, launched as two kernels.
// ---------------------------------------------------------------------------
template <int MB, int TG, int WB, bool SPLIT>
__device__ __forceinline__ void wide_body(
    const uint16_t* __restrict__ x, const float* __restrict__ s, const int8_t* __restrict__ wq,
    const float* __restrict__ wscale, int M, int N, int K, int tiles, int P, int U,
    int8_t* __restrict__ qx, float* __restrict__ sx, int32_t* __restrict__ partials,
    uint32_t* __restrict__ flags, uint16_t* __restrict__ y, int32_t* __restrict__ acc_out,
    WaitCtl wc) {
  using C = Wide<MB, TG, WB == 4 ? 2 : 1>;
  extern __shared__ __align__(16) char smem[];
  char* slots = smem;
  int32_t* red = reinterpret_cast<int32_t*>(smem + C::SLOTS);
  int* sync = reinterpret_cast<int*>(smem + C::SLOTS + C::RED);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G0 = gridDim.x, b = blockIdx.x;
  // With the token-block split, workgroups b and b + 8 (one XCD) take the two
  // halves (MB blocks each) of the token blocks of range r; otherwise range r
  // is workgroup r and takes all MB blocks.
  const int G = SPLIT ? G0 >> 1 : G0;
  const int r = SPLIT ? (b & 7) | ((b >> 4) << 3) : b;
  const int tb0 = SPLIT ? ((b >> 3) & 1) * MB : 0;
  const int mlo = tb0 * 16, mhi = SPLIT ? min(M, (tb0 + MB) * 16) : M;
  const int i0 = range_start(r, U, G);
  const int n = range_start(r + 1, U, G) - i0;
  const int nch = (K + 63) >> 6;
  if (tid < kSyncWords) sync[tid] = 0;  // ordered before use by barrier (1)

  if (wave < kS) {
    wide_streamer<MB, TG, WB, SPLIT>(wq, qx, M, K, tiles, nch, P, i0, n, wave, lane, b < M, tb0,
                                     slots, red, sync, wc);
    return;
  }

  // ---- helpers
  const int ht = tid - 64 * kS;
  uint32_t e;
  if (!wide_rows_and_gate<SPLIT>(x, s, M, K, b, G0, n, mlo, mhi, ht, wave - kS, lane, qx, sx, flags,
                                 sync, e, wc))
    return;
  wide_epilogue<MB, TG, WB, SPLIT>(wscale, sx, M, N, P, U, G, r, b, tb0, i0, n, e, ht, lane, red,
                                   sync, partials, flags, y, acc_out, wc);
}

#define QUASAR_WIDE_PARAMS                                                                   \
  const uint16_t *__restrict__ x, const float *__restrict__ s, const int8_t *__restrict__ wq, \
      const float *__restrict__ wscale, int M, int N, int K, int tiles, int P, int U,       \
      int8_t *__restrict__ qx, float *__restrict__ sx, int32_t *__restrict__ partials,     \
      uint32_t *__restrict__ flags, uint16_t *__restrict__ y, int32_t *__restrict__ acc_out, \
      WaitCtl wc
#define QUASAR_WIDE_ARGS x, s, wq, wscale, M, N, K, tiles, P, U, qx, sx, partials, flags, y, acc_out, wc

template <int MB, int TG>
__global__ __launch_bounds__(kThreads) void w8a8_linear_wide_kernel(QUASAR_WIDE_PARAMS) {
  wide_body<MB, TG, 8, false>(QUASAR_WIDE_ARGS);
}

template <int MB, int TG>
__global__ __launch_bounds__(kThreads) void w4a8_linear_wide_kernel(QUASAR_WIDE_PARAMS) {
  wide_body<MB, TG, 4, false>(QUASAR_WIDE_ARGS);
}

// The token-block split (groups of TG = 2 or 3 tiles, MB of the 2 MB token
// blocks per workgroup): its own kernels, so that the unsplit ones keep their
// constants.
template <int MB, int TG>
__global__ __launch_bounds__(kThreads) void w8a8_linear_wide_split_kernel(QUASAR_WIDE_PARAMS) {
  wide_body<MB, TG, 8, true>(QUASAR_WIDE_ARGS);
}

template <int MB, int TG>
__global__ __launch_bounds__(kThreads) void w4a8_linear_wide_split_kernel(QUASAR_WIDE_PARAMS) {
  wide_body<MB, TG, 4, true>(QUASAR_WIDE_ARGS);
}
#undef QUASAR_WIDE_PARAMS
#undef QUASAR_WIDE_ARGS

template <int MB, int TG, int WB, bool SPLIT = false>
hipError_t launch_wide_mb(const WidePlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                          const float* w_scale, uint16_t* y, int32_t* acc_out, int8_t* qx,
                          float* sx, int32_t* partials, uint32_t* flags, const WaitCtl& wc,
                          hipStream_t st) {
  auto kernel = [] {
    if constexpr (SPLIT && WB == 4)
      return &w4a8_linear_wide_split_kernel<MB, TG>;
    else if constexpr (SPLIT)
      return &w8a8_linear_wide_split_kernel<MB, TG>;
    else if constexpr (WB == 4)
      return &w4a8_linear_wide_kernel<MB, TG>;
    else
      return &w8a8_linear_wide_kernel<MB, TG>;
  }();
  constexpr int lds = Wide<MB, TG, WB == 4 ? 2 : 1>::LDS;
  static const hipError_t attr = hipFuncSetAttribute(
      reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize, lds);
  if (attr != hipSuccess) return attr;
  kernel<<<dim3(p.grid), dim3(kThreads), lds, st>>>(x, s, wq, w_scale, (int)p.M, (int)p.N,
                                                    (int)p.K, p.tiles, p.P, p.U, qx, sx, partials,
                                                    flags, y, acc_out, wc);
  return hipGetLastError();
}

template <int TG, int WB>
hipError_t launch_wide_tg(const WidePlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                          const float* w_scale, uint16_t* y, int32_t* acc_out, int8_t* qx,
                          float* sx, int32_t* partials, uint32_t* flags, const WaitCtl& wc,
                          hipStream_t st) {
#define QUASAR_WIDE_CASE(B)                                                                  \
  case B:                                                                                    \
    if constexpr (WB == 8 || B <= kWideMaxMbW4)                                              \
      return launch_wide_mb<B, TG, WB>(p, x, s, wq, w_scale, y, acc_out, qx, sx, partials,   \
                                       flags, wc, st);                                       \
    return hipErrorInvalidValue;
  switch (p.mbl) {
    QUASAR_WIDE_CASE(1)
    QUASAR_WIDE_CASE(2)
    QUASAR_WIDE_CASE(3)
    QUASAR_WIDE_CASE(4)
    QUASAR_WIDE_CASE(5)
    QUASAR_WIDE_CASE(6)
    QUASAR_WIDE_CASE(7)
    QUASAR_WIDE_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef QUASAR_WIDE_CASE
}

constexpr int wide_lds_of(int mb, int tg, int wb = 8) {
  return kS * wide_nbuf(mb, tg, wb == 4 ? 2 : 1) * (wb == 4 ? 2 : 1) * mb * 1024 +
         2 * kS * mb * 1024 + 256;
}
static_assert(wide_lds_of(6, 4) == Wide<6, 4>::LDS && wide_lds_of(3, 1) == Wide<3, 1>::LDS &&
                  wide_lds_of(6, 2, 4) == Wide<6, 2, 2>::LDS,
              "host LDS size matches the kernel's");

}  // namespace

// Tiles per group: groups of 4 tiles let each 16 x 64 activation fragment
// serve 4 tiles (a quarter of the code bytes per weight byte), but leave a
// linear with few tiles with fewer groups than workgroups, so that a group's
// K range is split across several workgroups that must hand INT32 partial
// sums to each other at the end of the launch.  With groups of one or two
// tiles each workgroup instead reads the whole code matrix per group, at the
// L2 read rate of contiguous 1 KB fragments.  Measured on MI355X (16 to 128
// tokens, K = 4096 unless stated; us per launch):
//   * up to 2 tiles per CU (QKV, O): the smallest group that gives at most one
//     group per CU, launched one group per workgroup (wide_launch_grid), so no
//     K range is split: 4096 -> 6144 at 48 and 96 tokens 14.2 -> 13.2 and
//     17.5 -> 16.5, 4096 -> 8192 at 48 tokens 16.4 -> 13.7, against single
//     tiles on every CU;
//   * 2 to 4 tiles per CU: pairs on every CU up to 64 tokens (4096 -> 12288 at
//     48 tokens 20.8 -> 17.4), beyond that groups of 4, one per workgroup (at
//     96 tokens 24.5 -> 21.6), against groups of 4 on every CU;
//   * up to 8 tiles per CU at up to 32 tokens: pairs on every CU (gate_up at
//     16 tokens 23.3 -> 20.9);
//   * K > 8192 (down): pairs of tiles on every CU, each K range split in two
//     (down at 48 and 96 tokens: 20.0 and 26.0 against 21.3 and 29.5 for
//     single tiles and 24.7 and 33.1 for one pair per workgroup);
//   * beyond 4 tiles per CU from 48 to 96 tokens (3 to 6 token blocks):
//     groups of 6 tiles, one per CU for gate_up (no K range split), with two
//     items in flight per streamer: gate_up at 48, 64, 80 and 96 tokens 26.0,
//     28.5, 31.3, 32.8 -> 22.7, 24.2, 26.6, 27.9; the LM head at 64 and 96
//     tokens 131.1 -> 126.1 and 152.5 -> 148.6; 4-bit gate_up at 48 and 96
//     tokens 20.6 -> 16.9 and 27.7 -> 23.9, its LM head 78.9 -> 74.6 and
//     117.5 -> 108.5;
//     below 48 tokens the same with 4-bit weights (gate_up at 16 and 32 tokens
//     16.5 -> 15.1 and 20.1 -> 16.2) and at 32 tokens up to 8 tiles per CU
//     with INT8 (gate_up 23.7 -> 22.6; at 16 tokens pairs stay faster, 20.3
//     against 21.7);
//   * beyond (the LM head above 96 tokens or with INT8 below 48 tokens, down
//     at 128 tokens): groups of 4 on every CU.
// Sharing each fragment among 16 tiles through LDS no longer paid once
// fragments were contiguous: 164 against 163 us on the 4096 -> 151936 LM head
// at 96 tokens, 206 against 183 at 128.
// Token-block split: at 64 tokens and more, up to one tile pair per range of
// a full grid, two workgroups of one XCD share each group of tiles and take
// half of the token blocks each, so each reads half the code matrix while the
// pair's weights come from HBM once and from L2 for the second reader; every
// range owns one whole pair (no K range split).  Measured on MI355X (us per
// launch, against the tile-group rule below, bit-identical outputs):
//   * K <= 8192: 4096 -> 4096 at 64, 96 and 128 tokens 13.2 -> 12.2,
//     14.7 -> 13.5 and 16.2 -> 15.1; 4096 -> 2048 at 96 tokens 14.1 -> 13.1;
//     4-bit weights at 96 tokens 13.5 -> 12.1;
//   * K > 8192 only with 256 tiles from 96 tokens (down at 96 tokens
//     26.0 -> 25.4, 4-bit 22.3 -> 20.9) or beyond 96 x 12288 codes (down at
//     128 tokens 33.7 -> 28.0): with fewer tiles or at 64 tokens the K-split
//     pairs of every CU stay faster (12288 -> 2048 at 96 tokens 21.5 against
//     24.2).
// Between 1 and 1.5 tiles per CU (QKV) the ranges take groups of 3 tiles
// (K <= 8192): 4096 -> 6144 at 64, 96 and 128 tokens 14.5 -> 14.0, 16.5 ->
// 16.0 and 18.2 -> 17.7; with 4-bit weights only from 96 tokens (14.9 ->
// 13.7; at 64 tokens 12.2 -> 13.0).
// Returns the tiles per group of the split (2 or 3), or 0 for no split.
int wide_token_split(int64_t M, int64_t N, int64_t K, int grid, int wbits) {
  const int64_t mb = (M + 15) / 16, tiles = (N + 15) / 16;
  const int64_t pairs = (tiles + 1) / 2, triples = (tiles + 2) / 3;
  const int64_t g = grid > 0 ? grid : kWideMaxGrid;
  if (mb < 4 || mb % 2 != 0) return 0;
  if (tiles <= g && pairs % 8 == 0 && 2 * pairs >= M &&
      (K <= 8192 || (tiles == g && mb >= 6) || M * K > 96 * 12288))
    return 2;
  if (tiles > g && 2 * tiles <= 3 * g && triples % 8 == 0 && 2 * triples >= M && K <= 8192 &&
      (wbits != 4 || mb >= 6))
    return 3;
  return 0;
}

int wide_tiles_per_group(int64_t M, int64_t N, int64_t K, int grid, int wbits) {
  const int64_t tiles = (N + 15) / 16, mb = (M + 15) / 16;
  const int64_t g = grid > 0 ? grid : kWideMaxGrid;
  if (M * K > 96 * 12288) return kMaxTG;
  if (K > 8192) return tiles <= 2 * g ? 2 : kMaxTG;
  if (tiles <= g) return 1;
  if (tiles <= 2 * g) return 2;
  if (tiles < 4 * g) return M <= 64 ? 2 : kMaxTG;
  if (tiles > 4 * g && mb <= 6 && (mb >= 3 || wbits == 4 || (mb == 2 && tiles <= 8 * g)))
    return kWideTG;
  if (tiles <= 8 * g && M <= 32) return 2;
  return kMaxTG;
}

WidePlan plan_wide(int64_t M, int64_t N, int64_t K, int grid, int wbits) {
  WidePlan p{};
  p.M = M;
  p.N = N;
  p.K = K;
  p.wb = wbits == 4 ? 4 : 8;
  p.mb = (int)((M + 15) / 16);
  const int split_tg = wide_token_split(M, N, K, grid, p.wb);
  p.ms = split_tg ? 2 : 1;
  p.mbl = p.mb / p.ms;
  p.tg = split_tg ? split_tg : wide_tiles_per_group(M, N, K, grid, p.wb);
  p.tiles = (int)((N + 15) / 16);
  p.nch = (int)((K + 63) / 64);
  p.groups = (p.tiles + p.tg - 1) / p.tg;
  // items of 4 weight blocks: 64-wide K chunks (INT8), pairs of them (4-bit)
  const int nwc = p.wb == 4 ? (int)(K / 128) : p.nch;
  p.P = (nwc + kS - 1) / kS;
  p.U = p.groups * p.P;
  p.grid = grid;
  p.lds = wide_lds_of(p.mbl, p.tg, p.wb);
  size_t off = kFlagHeaderBytes;  // the flag header (quasar_sync.hpp) comes first
  p.off_qx = off;  // fragment-major codes: 1 KB per 16-token block and 64-wide K chunk
  off = align_up(off + (size_t)p.mb * p.nch * 1024, kWsAlign);
  p.off_sx = off;
  off = align_up(off + (size_t)M * sizeof(float), kWsAlign);
  p.off_partials = off;
  off = align_up(off + (size_t)kWideMaxGrid * (p.tg > kMaxTG ? p.tg : kMaxTG) * p.mb * 1024,
                 kWsAlign);
  p.bytes = off;
  return p;
}

const char* wide_kernel_name(int mb, int tg, int wbits, bool split) {
  // "w8a8_linear_wide_kernel<MB, TG>" / "w4a8_linear_wide_kernel<MB, TG>" (TG 1, 2, 4), and
  // "w8a8_linear_wide_split_kernel<MB, TG>" / "w4a8_..." (TG 2, 3)
  static const std::vector<std::string> names = [] {
    std::vector<std::string> v;
    for (const char* k : {"w8a8_linear_wide_kernel<", "w4a8_linear_wide_kernel<",
                          "w8a8_linear_wide_split_kernel<", "w4a8_linear_wide_split_kernel<"})
      for (int t : {1, 2, 3, kMaxTG, kWideTG})
        for (int b = 1; b <= 8; ++b)
          v.push_back(std::string(k) + std::to_string(b) + ", " + std::to_string(t) + ">");
    return v;
  }();
  const int ki = (split ? 2 : 0) + (wbits == 4 ? 1 : 0);
  const int ti = tg <= 1 ? 0 : (tg == 2 ? 1 : (tg == 3 ? 2 : (tg == kMaxTG ? 3 : 4)));
  mb = mb < 1 ? 1 : (mb > 8 ? 8 : mb);
  return names[(ki * 5 + ti) * 8 + mb - 1].c_str();
}

bool wide_w4_supported(int64_t M) { return (M + 15) / 16 <= kWideMaxMbW4; }

#define QUASAR_WIDE_LAUNCH_ARGS p, x, s, wq, w_scale, y, acc_out, qx, sx, partials, flags, wc, st
hipError_t launch_wide(const WidePlan& p, const uint16_t* x, const float* s, const int8_t* wq,
                       const float* w_scale, uint16_t* y, int32_t* acc_out, void* workspace,
                       hipStream_t st) {
  char* ws = static_cast<char*>(workspace);
  int8_t* qx = reinterpret_cast<int8_t*>(ws + p.off_qx);
  float* sx = reinterpret_cast<float*>(ws + p.off_sx);
  int32_t* partials = reinterpret_cast<int32_t*>(ws + p.off_partials);
  uint32_t* flags = reinterpret_cast<uint32_t*>(ws);
  const WaitCtl wc = wait_ctl_for_current_device();
  if (!wc.status) return hipErrorInvalidSymbol;
  if (p.ms == 2) {  // token-block split: groups of 2 or 3 tiles, 2, 3 or 4 blocks per workgroup
#define QUASAR_SPLIT_ARGS p, x, s, wq, w_scale, y, acc_out, qx, sx, partials, flags, wc, st
#define QUASAR_SPLIT_TG(T)                                                                  \
  switch (p.mbl) {                                                                          \
    case 2:                                                                                 \
      return p.wb == 4 ? launch_wide_mb<2, T, 4, true>(QUASAR_SPLIT_ARGS)                   \
                       : launch_wide_mb<2, T, 8, true>(QUASAR_SPLIT_ARGS);                  \
    case 3:                                                                                 \
      return p.wb == 4 ? launch_wide_mb<3, T, 4, true>(QUASAR_SPLIT_ARGS)                   \
                       : launch_wide_mb<3, T, 8, true>(QUASAR_SPLIT_ARGS);                  \
    case 4:                                                                                 \
      return p.wb == 4 ? hipErrorInvalidValue : launch_wide_mb<4, T, 8, true>(QUASAR_SPLIT_ARGS); \
    default:                                                                                \
      return hipErrorInvalidValue;                                                          \
  }
    if (p.tg == 2) QUASAR_SPLIT_TG(2)
    if (p.tg == 3) QUASAR_SPLIT_TG(3)
    return hipErrorInvalidValue;
#undef QUASAR_SPLIT_TG
#undef QUASAR_SPLIT_ARGS
  }
  if (p.wb == 4) {
    if (p.tg == 1)
      return launch_wide_tg<1, 4>(p, x, s, wq, w_scale, y, acc_out, qx, sx, partials, flags, wc, st);
    if (p.tg == 2)
      return launch_wide_tg<2, 4>(p, x, s, wq, w_scale, y, acc_out, qx, sx, partials, flags, wc, st);
    if (p.tg == kMaxTG)
      return launch_wide_tg<kMaxTG, 4>(p, x, s, wq, w_scale, y, acc_out, qx, sx, partials, flags,
                                       wc, st);
    if (p.tg == kWideTG) {
      switch (p.mbl) {
        case 1: return launch_wide_mb<1, kWideTG, 4>(QUASAR_WIDE_LAUNCH_ARGS);
        case 2: return launch_wide_mb<2, kWideTG, 4>(QUASAR_WIDE_LAUNCH_ARGS);
        case 3: return launch_wide_mb<3, kWideTG, 4>(QUASAR_WIDE_LAUNCH_ARGS);
        case 4: return launch_wide_mb<4, kWideTG, 4>(QUASAR_WIDE_LAUNCH_ARGS);
        case 5: return launch_wide_mb<5, kWideTG, 4>(QUASAR_WIDE_LAUNCH_ARGS);
        case 6: return launch_wide_mb<6, kWideTG, 4>(QUASAR_WIDE_LAUNCH_ARGS);
        default: return hipErrorInvalidValue;
      }
    }
    return hipErrorInvalidValue;
  }
  if (p.tg == 1)
    return launch_wide_tg<1, 8>(p, x, s, wq, w_scale, y, acc_out, qx, sx, partials, flags, wc, st);
  if (p.tg == 2)
    return launch_wide_tg<2, 8>(p, x, s, wq, w_scale, y, acc_out, qx, sx, partials, flags, wc, st);
  if (p.tg == kMaxTG)
    return launch_wide_tg<kMaxTG, 8>(p, x, s, wq, w_scale, y, acc_out, qx, sx, partials, flags, wc,
                                     st);
  if (p.tg == kWideTG) {
    switch (p.mbl) {
      case 2: return launch_wide_mb<2, kWideTG, 8>(QUASAR_WIDE_LAUNCH_ARGS);
      case 3: return launch_wide_mb<3, kWideTG, 8>(QUASAR_WIDE_LAUNCH_ARGS);
      case 4: return launch_wide_mb<4, kWideTG, 8>(QUASAR_WIDE_LAUNCH_ARGS);
      case 5: return launch_wide_mb<5, kWideTG, 8>(QUASAR_WIDE_LAUNCH_ARGS);
      case 6: return launch_wide_mb<6, kWideTG, 8>(QUASAR_WIDE_LAUNCH_ARGS);
      default: return hipErrorInvalidValue;
    }
  }
  return hipErrorInvalidValue;
}
#undef QUASAR_WIDE_LAUNCH_ARGS

// Scratch of quasar_w8a8_linear_noalloc: the wide kernel's workspace (flag
// header, quantized rows, token scales, INT32 partials) in a file-scope device
// array, one per device, zero at load (so its flag header starts valid) and
// held until the process ends.  Host code never passes the array's name to a
// kernel: it takes the device address from hipGetSymbolAddress once per
// device and uses that.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

void* noalloc_scratch_for_current_device() {
  static std::mutex mu;
  static void* ptr[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptr[dev] = p;
  }
  return ptr[dev];
}

// Workgroups the wide kernel launches on the current device: one per compute
// unit, at most kWideMaxGrid; 0 if one workgroup does not fit a compute unit.
// Fixed per device for the life of the process (the workspace flags rely on
// every launch using the same grid).
int wide_grid_for_current_device() {
  static std::mutex mu;
  static int cache[64];
  static bool init[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> lock(mu);
  if (!init[dev]) {
    int cus = 0, occ = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
      cus = 0;
    // every instantiation has the same block size; the largest LDS decides
    int lds = 0;
    for (int mb = 1; mb <= 8; ++mb)
      for (int tg : {1, 2, kMaxTG})
        for (int wb : {8, 4}) {
          if (wb == 4 && mb > kWideMaxMbW4) continue;
          lds = wide_lds_of(mb, tg, wb) > lds ? wide_lds_of(mb, tg, wb) : lds;
        }
    auto kernel = &w8a8_linear_wide_kernel<6, kMaxTG>;
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, kernel, kThreads, lds) != hipSuccess)
      occ = 0;
    cache[dev] = occ >= 1 ? (cus < kWideMaxGrid ? cus : kWideMaxGrid) : 0;
    init[dev] = true;
  }
  return cache[dev];
}

int wide_launch_grid(const WidePlan& p) {
  const int dev = wide_grid_for_current_device();
  if (p.ms == 2) {
    // two workgroups per range, one range per pair of tiles; the pairs of an
    // XCD need a grid that is a multiple of 16 (fewer ranges split K)
    if (2 * p.groups <= dev) return 2 * p.groups;
    const int g16 = dev / 16 * 16;
    return g16 >= p.M ? g16 : 0;
  }
  // one group per workgroup where the groups fit the device's grid and K is
  // not split (wide_tiles_per_group); still one workgroup per token row
  if (dev > 0 && p.K <= 8192 && p.groups <= dev && p.groups >= p.M) return p.groups;
  return dev;
}

}  // namespace quasar
