// Diagnostic kernel: a plain device-to-device copy with 16-byte vector loads
// and stores.  It is the reference workload for reading hardware byte
// counters: a copy of B bytes fetches and writes exactly B bytes.
#include "quasar_device.hpp"
#include "quasar_internal.hpp"

namespace quasar {
namespace {

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

}  // namespace

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
