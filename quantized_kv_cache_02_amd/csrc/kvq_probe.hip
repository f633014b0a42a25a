// kvq_probe.hip -- libkvq_probe (include/kvq_probe.h): a plain streaming read,
// as the floor the decode's KV reads are compared with: the same non-temporal
// 16-byte loads, every byte read once, no arithmetic beyond an XOR that keeps
// the loads alive.  Built as its own library; the attention path never loads it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvq_probe.h"

namespace kvq {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kUnroll = 8;  // 16-byte loads in flight per thread

// Workgroup w reads the w-th contiguous slice of the n16 16-byte units.
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4_t* __restrict__ src, int64_t n16,
                                                          u32x4_t* __restrict__ sink) {
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t beg = (int64_t)blockIdx.x * per;
  const int64_t end = beg + per < n16 ? beg + per : n16;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (int64_t i = beg + threadIdx.x; i < end; i += 256 * kUnroll) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t j = i + 256 * u;
      v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u];
  }
  // a store only for one XOR pattern in 2^64, so the loads cannot be dropped
  if (acc[0] == 0x9E3779B9u && acc[1] == 0x7F4A7C15u) sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = acc;
}

}  // namespace
}  // namespace kvq

extern "C" int kvq_stream_read(const void* src, size_t bytes, int32_t workgroups, void* sink,
                               void* stream) {
  if (src == nullptr || sink == nullptr || bytes % 16 != 0 || workgroups < 1 || workgroups > 65535)
    return KVQ_EINVAL;
  if (bytes == 0) return KVQ_OK;
  hipLaunchKernelGGL(kvq::stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     static_cast<hipStream_t>(stream), static_cast<const kvq::u32x4_t*>(src),
                     (int64_t)(bytes / 16), static_cast<kvq::u32x4_t*>(sink));
  return hipGetLastError() == hipSuccess ? KVQ_OK : KVQ_EHIP;
}
