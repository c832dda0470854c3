// Read-bandwidth probe: a measurement aid for the roofline of the attention kernels, not part of
// the attention path. It streams a buffer with the 16-byte nontemporal loads the split kernel
// issues for its KV tiles, in the most favourable order measured on MI355X (each workgroup reads
// one contiguous 1 MiB range, 16 KiB per step with four loads in flight per lane: 7.0-7.1 TB/s
// over 4 GiB, where a grid-stride order reached 6.1-6.2) and with no compute, so its rate is the
// practical ceiling of a read stream on the device.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kv_attn.h"

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kProbeThreads = 256;
constexpr uint64_t kChunk16 = uint64_t(KV_ATTN_PROBE_CHUNK) / 16;  // 16-byte words per workgroup

__device__ __forceinline__ uint32_t fold(const u32x4_t* p) {
  const u32x4_t x = __builtin_nontemporal_load(p);
  return x[0] ^ x[1] ^ x[2] ^ x[3];
}

// Workgroup w reads words [w * kChunk16, min((w + 1) * kChunk16, n16)). The words' XOR is
// compared with a constant so that the loads stay live; the store it guards writes *sink (a
// value the caller ignores) only in the case that the XOR matches.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const u32x4_t* src, uint64_t n16,
                                                                   uint32_t* sink) {
  const uint64_t begin = uint64_t(blockIdx.x) * kChunk16;
  const uint64_t end = begin + kChunk16 < n16 ? begin + kChunk16 : n16;
  uint64_t i = begin + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * kProbeThreads < end; i += 4 * kProbeThreads)
    acc ^= fold(src + i) ^ fold(src + i + kProbeThreads) ^ fold(src + i + 2 * kProbeThreads) ^
           fold(src + i + 3 * kProbeThreads);
  for (; i < end; i += kProbeThreads) acc ^= fold(src + i);
  if (acc == 0x9e3779b9u) *sink = acc;
}

}  // namespace

extern "C" kv_attn_status kv_attn_read_probe(const void* src, uint64_t bytes, uint32_t* sink,
                                             void* stream) {
  if (src == nullptr || sink == nullptr) return KV_ATTN_ERR_NULL;
  if (bytes == 0 || (bytes & 15u) != 0 || (reinterpret_cast<uintptr_t>(src) & 15u) != 0)
    return KV_ATTN_ERR_UNSUPPORTED;
  const uint64_t grid = (bytes + KV_ATTN_PROBE_CHUNK - 1) / KV_ATTN_PROBE_CHUNK;
  if (grid > 0x7fffffffu) return KV_ATTN_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(read_probe_kernel, dim3(uint32_t(grid)), dim3(kProbeThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), reinterpret_cast<const u32x4_t*>(src),
                     bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? KV_ATTN_OK : KV_ATTN_ERR_HIP;
}
