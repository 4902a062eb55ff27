// Streaming-read probe: the achievable HBM read rate on this GPU, measured with the same kind of
// load the decode kernel streams KV with (16-byte non-temporal loads, whole 1 KiB rows per wave
// instruction).  Not part of the paged path; the benchmark reports decode bandwidth against it
// beside the published peak.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 16;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(
    const u32x4_t* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = tid;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  sink[tid] = acc;
}

hipError_t launch_hbm_probe(const void* src, size_t bytes, uint32_t* sink, int num_workgroups,
                            hipStream_t stream) {
  hipLaunchKernelGGL(hbm_read_probe_kernel, dim3(num_workgroups), dim3(kProbeThreads), 0, stream,
                     static_cast<const u32x4_t*>(src), static_cast<int64_t>(bytes / 16), sink);
  return hipGetLastError();
}

}  // namespace pa
