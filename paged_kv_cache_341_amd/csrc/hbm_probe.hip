// Streaming-read probe: the achievable HBM read rate on this GPU, measured with the load the
// decode kernel streams KV with (16-byte non-temporal loads, whole 1 KiB rows per wave
// instruction).  Each wave reads its own contiguous range, 16 KiB (16 rows) per batch; the
// benchmark takes the best of a few grid sizes, so the figure is the best plain streaming rate,
// an upper bound for any kernel's reads.  Not part of the paged path; the benchmark reports
// decode bandwidth against it beside the published peak.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

constexpr int kProbeThreads = 256;
constexpr int kProbeUnroll = 16;

__global__ __launch_bounds__(kProbeThreads) void hbm_read_probe_kernel(
    const u32x4_t* __restrict__ src, int64_t n16, uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x % kWave;
  const int64_t waves = static_cast<int64_t>(gridDim.x) * (kProbeThreads / kWave);
  const int64_t w = static_cast<int64_t>(blockIdx.x) * (kProbeThreads / kWave) + threadIdx.x / kWave;
  constexpr int64_t kBatch = static_cast<int64_t>(kProbeUnroll) * kWave;   // chunks per batch
  const int64_t per_wave = n16 / waves / kBatch * kBatch;                  // whole batches
  const u32x4_t* p = src + w * per_wave;
  uint32_t acc = 0;
  for (int64_t i = lane; i < per_wave; i += kBatch) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * kWave);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  // what the whole batches left over, spread over all lanes
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * kProbeThreads + threadIdx.x;
  for (int64_t i = waves * per_wave + tid; i < n16;
       i += static_cast<int64_t>(gridDim.x) * kProbeThreads) {
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
