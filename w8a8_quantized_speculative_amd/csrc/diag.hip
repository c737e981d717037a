// Diagnostics of libquasar: the device status word that reports bounded waits
// that gave up (see quasar_sync.hpp), the forced-expiry test hook, and a plain
// device-to-device copy with 16-byte vector loads and stores -- the reference
// workload for reading hardware byte counters (a copy of B bytes fetches and
// writes exactly B bytes).
#include <atomic>
#include <mutex>

#include "quasar_device.hpp"
#include "quasar_internal.hpp"
#include "quasar_sync.hpp"

namespace quasar {

// One word per device (each device that loads the library holds its own copy).
__device__ uint32_t g_wait_status;

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_status_mutex;
uint32_t* g_status_ptr[kMaxDevices];
std::atomic<bool> g_forced{false};

uint32_t* status_word_for_device(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_status_mutex);
  if (!g_status_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(g_wait_status)) != hipSuccess) return nullptr;
    g_status_ptr[dev] = static_cast<uint32_t*>(p);
  }
  return g_status_ptr[dev];
}

__global__ __launch_bounds__(256) void stream_copy_kernel(const v4i* __restrict__ src,
                                                          v4i* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const v4i a = __builtin_nontemporal_load(src + i);
    const v4i b = __builtin_nontemporal_load(src + i + stride);
    const v4i c = __builtin_nontemporal_load(src + i + 2 * stride);
    const v4i d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// Plain streaming read: each workgroup reads one contiguous range with
// 16-byte streaming (nt) loads, four per lane in flight, folded into one word
// so the loads are kept: the reference rate for a read-only stream.  Measured
// on MI355X: 7.07 TB/s over 1 GiB; one launch per buffer, back to back, 4.1,
// 4.9, 5.8, 6.4 and 6.8 TB/s over 16.8, 25.2, 50.3, 100.7 and 622 MB.
// Grid-stride order gave 5.2-5.9 TB/s over 1 GiB, and plain (non-streaming)
// loads about 6.1 TB/s.
__global__ __launch_bounds__(256) void stream_read_kernel(const v4i* __restrict__ src, size_t n16,
                                                          uint32_t* __restrict__ sink) {
  const size_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const size_t b0 = (size_t)blockIdx.x * per;
  const size_t b1 = b0 + per < n16 ? b0 + per : n16;
  v4i acc = {0, 0, 0, 0};
  size_t i = b0 + threadIdx.x;
  for (; i + 3 * 256 < b1; i += 4 * 256) {
    const v4i a = __builtin_nontemporal_load(src + i);
    const v4i b = __builtin_nontemporal_load(src + i + 256);
    const v4i c = __builtin_nontemporal_load(src + i + 512);
    const v4i d = __builtin_nontemporal_load(src + i + 768);
    acc ^= a ^ b ^ c ^ d;
  }
  for (; i < b1; i += 256) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t v = (uint32_t)(acc.x ^ acc.y ^ acc.z ^ acc.w);
  if (v == 0x9e3779b9u) sink[blockIdx.x] = v;  // keeps the loads; practically never stores
}

// Zero fill of a workspace's flag header by a kernel (not a memset node), so
// that it can sit inside a captured graph.
__global__ __launch_bounds__(256) void zero_words_kernel(uint32_t* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

}  // namespace

WaitCtl wait_ctl_for_current_device() {
  int dev = -1;
  WaitCtl w{nullptr, 0u, kSpinLdsDefault, kSpinGlobalDefault};
  if (hipGetDevice(&dev) != hipSuccess) return w;
  w.status = status_word_for_device(dev);
  if (g_forced.load()) {
    w.bias = kForcedBias;
    w.spin_lds = kSpinForced;
    w.spin_global = kSpinForced;
  }
  return w;
}

void set_forced_wait_expiry(bool on) { g_forced.store(on); }

hipError_t read_and_clear_status(uint32_t* bits) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (!status_word_for_device(dev)) return hipErrorInvalidSymbol;
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_status_mutex);
  uint32_t v = 0;
  e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_wait_status), sizeof(v), 0, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return e;
  const uint32_t zero = 0;
  e = hipMemcpyToSymbol(HIP_SYMBOL(g_wait_status), &zero, sizeof(zero), 0, hipMemcpyHostToDevice);
  if (e != hipSuccess) return e;
  *bits = v;
  return hipSuccess;
}

hipError_t launch_zero_flag_header(void* workspace, hipStream_t st) {
  zero_words_kernel<<<dim3(1), dim3(256), 0, st>>>(static_cast<uint32_t*>(workspace),
                                                   (int)(kFlagHeaderBytes / sizeof(uint32_t)));
  return hipGetLastError();
}

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* sink, hipStream_t st) {
  const size_t n16 = bytes / 16;
  // up to eight workgroups per compute unit, each with at least 16 KB to read
  // (within 3% of the fastest grid at every size measured up to 622 MB); two
  // per compute unit from 512 MB on (7.07 against 6.7-6.9 TB/s over 1 GiB)
  size_t blocks = (n16 + 1023) / 1024;
  const size_t cap = (bytes >= ((size_t)512 << 20) ? 2 : 8) * (size_t)kNumCU;
  if (blocks > cap) blocks = cap;
  if (blocks == 0) return hipSuccess;
  stream_read_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(static_cast<const v4i*>(src),
                                                                   n16, sink);
  return hipGetLastError();
}

hipError_t launch_stream_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4 * (size_t)kNumCU) blocks = 4 * (size_t)kNumCU;
  if (blocks == 0) return hipSuccess;
  stream_copy_kernel<<<dim3((unsigned)blocks), dim3(256), 0, st>>>(
      static_cast<const v4i*>(src), static_cast<v4i*>(dst), n16);
  return hipGetLastError();
}

}  // namespace quasar
