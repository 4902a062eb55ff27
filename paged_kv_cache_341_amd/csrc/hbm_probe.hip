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

// Matrix-core probe: the achievable dense bf16 MFMA rate on this GPU under load, measured with
// the instruction the prefill and shared-prefix kernels use (v_mfma_f32_32x32x16_bf16).  Every
// wave of 512-lane workgroups runs `iters` rounds of four independent accumulation chains on
// register operands (no memory traffic), then writes one folded value per lane to `sink`.  Not
// part of the paged path; the benchmark reports prefill MFMA rates against it beside the
// published peak.
constexpr int kMfmaProbeThreads = 512;
constexpr int kMfmaProbeChains = 4;

__global__ __launch_bounds__(kMfmaProbeThreads) void mfma_probe_kernel(float* __restrict__ sink,
                                                                        int iters) {
  bf16x8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = static_cast<__bf16>(1e-3f * static_cast<float>((threadIdx.x + i) & 63));
    b[i] = static_cast<__bf16>(2e-3f * static_cast<float>(i));
  }
  f32x16_t acc[kMfmaProbeChains];
#pragma unroll
  for (int c = 0; c < kMfmaProbeChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[c][v] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < kMfmaProbeChains; ++c)
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kMfmaProbeChains; ++c)
#pragma unroll
    for (int v = 0; v < 16; ++v) s += acc[c][v];
  sink[static_cast<size_t>(blockIdx.x) * kMfmaProbeThreads + threadIdx.x] = s;
}

hipError_t launch_mfma_probe(float* sink, int num_workgroups, int iters, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(num_workgroups), dim3(kMfmaProbeThreads), 0, stream,
                     sink, iters);
  return hipGetLastError();
}

}  // namespace pa
