// Cross-workgroup hand-offs and bounded waits of libquasar's persistent
// kernels, and the device status word that reports a wait that gave up.
//
// Protocol (every kernel that hands data from one workgroup to another within a
// launch follows it):
//   * writer: the handed-off data is stored with agent-scope stores (the sc1
//     cache policy: written through to the device's coherence point); the
//     wavefront waits until all its stores have completed, and only then
//     stores the flag, also agent-scope;
//   * reader: one wavefront polls the flag(s) with agent-scope loads, then
//     tells the other wavefronts of its workgroup through an LDS counter; every
//     read of the handed-off data comes after that and is itself an
//     agent-scope load (sc1), which never returns a stale cached copy.
// Each access that crosses workgroups is thus coherent on its own, and the
// order comes from the completion wait on the writer side and the flag seen
// on the reader side.  No cache-wide fence is used: on MI355X an agent-scope
// release fence writes back the XCD's whole L2 and an acquire fence
// invalidates it, which measured +14 us and +7 us per launch of a 96-token
// 4096 -> 6144 linear, while agent-scope loads of the handed-off data still
// hit in L2 (the same launch within 1%).
// Flags live in the caller's workspace (never in library memory), so calls on
// different streams with different workspaces are independent.  Each flag word
// belongs to one workgroup and only grows: a launch reads its own word first
// and every target is relative to that value, so the words need to be equal
// (e.g. all zero) when the workspace is first used and never need a reset.
// A launch with fewer workgroups than slots advances the slots beyond its grid
// too, so the words stay equal across launches of different grids.
//
// Every wait is bounded.  A wait that gives up sets a bit of the device status
// word and the kernel continues (with undefined outputs for that call) instead
// of hanging; quasar_device_check() reads and clears the word.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace quasar {

// Status bits (also in include/quasar.h).
constexpr uint32_t kWaitLds = 1u;        // an in-workgroup (LDS counter) wait
constexpr uint32_t kWaitRows = 2u;       // a wait for other workgroups' quantized rows
constexpr uint32_t kWaitPartials = 4u;   // a wait for other workgroups' INT32 partial sums
constexpr uint32_t kWaitChain = 8u;      // a wait for an earlier link of a chained call

// What a kernel needs to bound and report its waits.  `bias` is 0 except under
// the forced-expiry test hook, which adds it to every wait target so that no
// target is reachable, with a small spin bound: every wait then gives up and
// every kernel still exits normally.
struct WaitCtl {
  uint32_t* status;  // the device status word
  uint32_t bias;
  int spin_lds;      // polls of an LDS counter
  int spin_global;   // polls of a flag in global memory
};

constexpr int kSpinLdsDefault = 1 << 22;
constexpr int kSpinGlobalDefault = 1 << 20;
constexpr int kSpinForced = 64;
constexpr uint32_t kForcedBias = 1u << 30;

// Host: the control block for a launch on the current device (status word of
// that device, the test hook's bias and bounds).  status == nullptr if the
// word cannot be located (the launcher then reports a HIP error).
WaitCtl wait_ctl_for_current_device();
// Host: the forced-expiry test hook.
void set_forced_wait_expiry(bool on);
// Host: wait for the current device, read and clear its status word.
hipError_t read_and_clear_status(uint32_t* bits);

// The flag header at the start of every workspace that carries cross-workgroup
// flags: two flag words per workgroup slot, each alone in its 128-byte line.
// With 256 workgroups polling the same few lines, packed flags made every
// hand-off slower: spreading them cut about 2 us from each wide-window launch
// at 48 and 96 tokens, and 0.14 ms from a 145-link chain.
constexpr int kFlagSlots = 256;
constexpr int kFlagStride = 32;  // words between two flags
constexpr size_t kFlagHeaderBytes = 2 * kFlagSlots * kFlagStride * sizeof(uint32_t);

// Flag word of workgroup slot b in the first (set 0) or second (set 1) set.
__host__ __device__ __forceinline__ uint32_t* flag_word(uint32_t* header, int set, int b) {
  return header + (set * kFlagSlots + b) * kFlagStride;
}

__device__ __forceinline__ void note_expired(const WaitCtl& w, uint32_t bit) {
  __hip_atomic_fetch_or(w.status, bit, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ uint32_t load_flag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void store_flag(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Cache-policy bit of buffer loads for agent-scope (coherent) access: sc1.
constexpr int kCoherent = 16;

// Writer side, after the handed-off data has been stored (agent scope): wait
// until every memory operation of this wavefront has completed, so that the
// flag stored next is seen only after the data.
__device__ __forceinline__ void wait_stores_complete() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0); expcnt and lgkmcnt at their maxima (no wait)
  asm volatile("" ::: "memory");
}

// Reader side, after a poll succeeded: keeps the compiler from moving the
// data reads above the poll (they are agent-scope loads themselves).
__device__ __forceinline__ void after_poll() { asm volatile("" ::: "memory"); }

// Agent-scope loads of handed-off data.
__device__ __forceinline__ float load_coherent(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Signed distance of a growing 32-bit counter from a target (wrap-safe).
__device__ __forceinline__ bool reached(uint32_t v, uint32_t target) {
  return (int32_t)(v - target) >= 0;
}

// Bounded wait until an LDS counter reaches `target` (+ the test bias).
__device__ __forceinline__ void lds_wait_at_least(const int* p, int target, const WaitCtl& w) {
  const int t = target + (int)w.bias;
  for (int spin = 0;; ++spin) {
    if (__hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= t) break;
    if (spin >= w.spin_lds) {
      note_expired(w, kWaitLds);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  asm volatile("" ::: "memory");  // later LDS accesses stay below the wait
}

}  // namespace quasar
