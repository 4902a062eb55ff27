// KV append through a slot mapping, and copy-on-write whole-block copies, for gfx950.
//
// Append: a sequence grows into its current block (study-docs "PagedAttention & Continuous
// Batching", section "Block tables"); token t's K and V rows go to slot_mapping[t] =
// block * block_size + offset, negative slots being padding.  Copy-on-write: before a write
// into a shared block, a fresh block receives a copy of it (study-docs, section
// "Copy-on-write"; cloudmash "Batching and PagedAttention", section "Sharing blocks").
//
// Both are pure byte movement: every lane moves 16-byte chunks, consecutive lanes consecutive
// chunks, so each wave reads and writes whole 1 KiB runs of a row or block.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

constexpr int kCopyThreads = 256;

// One lane per 16-byte chunk of a (token, kv head) row, for K and V.
__global__ __launch_bounds__(kCopyThreads) void kv_append_kernel(
    char* __restrict__ k_cache, char* __restrict__ v_cache, const char* __restrict__ k_new,
    const char* __restrict__ v_new, const int64_t* __restrict__ slot_mapping,
    int64_t total_chunks, int chunks_per_row, int num_kv_heads, int block_size,
    int* __restrict__ zero_words, int num_zero_words) {
  if (blockIdx.x == 0 && static_cast<int>(threadIdx.x) < num_zero_words) zero_words[threadIdx.x] = 0;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
       i < total_chunks; i += stride) {
    const int64_t row = i / chunks_per_row;            // (token, head)
    const int c = static_cast<int>(i % chunks_per_row);
    const int64_t t = row / num_kv_heads;
    const int h = static_cast<int>(row % num_kv_heads);
    const int64_t slot = slot_mapping[t];
    if (slot < 0) continue;
    const int64_t b = slot / block_size;
    const int64_t o = slot % block_size;
    const int64_t dst = (((b * num_kv_heads + h) * block_size + o) * chunks_per_row + c) * 16;
    const int64_t src = i * 16;
    store16(k_cache + dst, load16(k_new + src));
    store16(v_cache + dst, load16(v_new + src));
  }
}

// One lane per 16-byte chunk of a block, for K and V: block pairs[p][1] of the destination
// pools becomes a copy of block pairs[p][0] of the source pools.  Copy-on-write passes the same
// pool as source and destination (a destination is never a source there, so the blocks read
// and written are distinct); a swap passes a device pool and a host pool the device can map.
__global__ __launch_bounds__(kCopyThreads) void block_copy_kernel(
    char* __restrict__ dst_k, char* __restrict__ dst_v, const char* __restrict__ src_k,
    const char* __restrict__ src_v, const int64_t* __restrict__ pairs, int64_t total_chunks,
    int64_t chunks_per_block) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kCopyThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kCopyThreads + threadIdx.x;
       i < total_chunks; i += stride) {
    const int64_t p = i / chunks_per_block;
    const int64_t c = i % chunks_per_block;
    const int64_t src = pairs[2 * p];
    const int64_t dst = pairs[2 * p + 1];
    const int64_t so = (src * chunks_per_block + c) * 16;
    const int64_t d = (dst * chunks_per_block + c) * 16;
    store16(dst_k + d, load16(src_k + so));
    store16(dst_v + d, load16(src_v + so));
  }
}

static unsigned grid_for(int64_t total) {
  const int64_t want = (total + kCopyThreads - 1) / kCopyThreads;
  return static_cast<unsigned>(std::min<int64_t>(want, 256 * 64));
}

hipError_t launch_append(const AppendArgs& a) {
  const int chunks_per_row = a.head_dim * a.elem_bytes / 16;
  const int64_t total = static_cast<int64_t>(a.num_tokens) * a.num_kv_heads * chunks_per_row;
  if (total == 0 && a.num_zero_words == 0) return hipSuccess;
  hipLaunchKernelGGL(kv_append_kernel, dim3(std::max(1u, grid_for(total))), dim3(kCopyThreads), 0,
                     a.stream, static_cast<char*>(a.k_cache), static_cast<char*>(a.v_cache),
                     static_cast<const char*>(a.k_new), static_cast<const char*>(a.v_new),
                     a.slot_mapping, total, chunks_per_row, a.num_kv_heads, a.block_size,
                     a.zero_words, a.num_zero_words);
  return hipGetLastError();
}

hipError_t launch_cow(const CowArgs& a) {
  const int64_t per_block = a.block_bytes / 16;
  const int64_t total = per_block * a.num_pairs;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(block_copy_kernel, dim3(grid_for(total)), dim3(kCopyThreads), 0, a.stream,
                     static_cast<char*>(a.dst_k), static_cast<char*>(a.dst_v),
                     static_cast<const char*>(a.src_k), static_cast<const char*>(a.src_v),
                     a.pairs, total, per_block);
  return hipGetLastError();
}

}  // namespace pa
