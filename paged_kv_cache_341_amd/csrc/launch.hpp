// Host-side launch descriptors shared by the C-ABI layer and the kernel translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace pa {

// How a sequence's units are cut into decode splits: c0 splits of s0 units, then c1 splits of
// s1 units, then splits of s2 units to the end, with s0 >= s1 >= s2 (a uniform plan has one
// size).  Split j covers units [start(j), start(j + 1)) of the sequence, clamped to its length.
// Every workgroup of split index j is launched after all of index j - 1, so shrinking sizes put
// the smallest pieces last.
struct SplitPlan {
  int s0, c0, s1, c1, s2;
  __host__ __device__ static SplitPlan uniform(int units) { return {units, 0, units, 0, units}; }
  __host__ __device__ int start(int j) const {
    const int a = j < c0 ? j : c0;
    const int b = j - c0 < 0 ? 0 : (j - c0 < c1 ? j - c0 : c1);
    const int c = j - c0 - c1 < 0 ? 0 : j - c0 - c1;
    return a * s0 + b * s1 + c * s2;
  }
  // number of splits that cover n units
  __host__ __device__ int count(int n) const {
    if (n <= 0) return 0;
    const int e0 = c0 * s0;
    if (n <= e0) return (n + s0 - 1) / s0;
    const int e1 = e0 + c1 * s1;
    if (n <= e1) return c0 + (n - e0 + s1 - 1) / s1;
    return c0 + c1 + (n - e1 + s2 - 1) / s2;
  }
  __host__ __device__ int max_units() const {
    int m = s2;
    if (c1 > 0 && s1 > m) m = s1;
    if (c0 > 0 && s0 > m) m = s0;
    return m;
  }
};

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  float* ws_ml;        // [S][Hq][nsplit_max][2]  (max in log2 units, sum)
  float* ws_acc;       // [S][Hq][nsplit_max][D]
  // Grouped decode (a prefix shared inside each group of sequences, done by the shared-prefix
  // kernel): per-sequence leading blocks to skip (null for plain decode), the slot where the
  // split kernel's partials start, and the keys per shared-prefix split.
  const int32_t* skip_blocks;
  int slot_base, shared_split_keys;
  int nsplit_tail;     // grid.y of the split kernel
  // Contiguous KV ([num_seqs][num_kv_heads][capacity][head_dim], no table) instead of a pool.
  bool contiguous;
  int capacity;
  // block_size: tokens per pool block.  The split walk goes in units of block_size tokens, or of
  // 16 tokens when blocks are smaller than 8 (each token's block is then looked up on its own)
  // and for contiguous KV; the plan counts units.
  int num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_blocks_per_seq;
  SplitPlan plan;
  int nsplit_max;
  float scale_log2;
  bool bf16;
  hipStream_t stream;
};

struct PrefillArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  const int32_t* query_start_loc;
  int num_chunks, total_q, max_q_len, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq;
  float scale_log2;
  hipStream_t stream;
};

struct AppendArgs {
  void* k_cache;
  void* v_cache;
  const void* k_new;
  const void* v_new;
  const int64_t* slot_mapping;
  int num_tokens, num_kv_heads, head_dim, block_size, elem_bytes;
  int* zero_words;               // optional: words set to 0 by the append launch (counters of a
  int num_zero_words;            // kernel that runs next on the same stream), at most 64
  hipStream_t stream;
};

// One launch of prefill chunks and decode splits together (bf16, D 128, B 16), after the append.
struct MixedArgs {
  // chunks
  void* chunk_out;
  const void* chunk_q;
  const int32_t* chunk_tables;
  const int32_t* chunk_seq_lens;
  const int32_t* query_start_loc;
  int num_chunks, chunk_max_blocks_per_seq;
  // decodes
  void* dec_out;
  const void* dec_q;
  const int32_t* dec_tables;
  const int32_t* dec_seq_lens;
  int num_seqs, dec_max_blocks_per_seq;
  SplitPlan plan;                // the decode splits, as pa_decode's plan
  int nsplit_max;
  float* ws_ml;
  float* ws_acc;
  int* queues;                   // two work counters, zero when the kernel starts
  // shared
  const void* k_cache;
  const void* v_cache;
  int num_q_heads, num_kv_heads, head_dim, num_workgroups;
  float scale_log2;
  hipStream_t stream;
};

// Whole-block copies from (src_k, src_v) to (dst_k, dst_v): copy-on-write within one pool, or
// swap between a device pool and a mapped host pool.
struct CowArgs {
  void* dst_k;
  void* dst_v;
  const void* src_k;
  const void* src_v;
  const int64_t* pairs;
  int num_pairs;
  int64_t block_bytes;
  hipStream_t stream;
};

hipError_t launch_decode(const DecodeArgs& a);

struct SharedPrefixArgs {
  float* ws_ml;
  float* ws_acc;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* group_start;    // [num_groups + 1]
  const int32_t* shared_blocks;  // [num_seqs]
  const int32_t* seq_lens;       // [num_seqs]
  int num_seqs, num_groups, num_q_heads, num_kv_heads, head_dim, max_blocks_per_seq;
  int row_tiles, nsplit_shared, split_keys, slot_base, nsplit_max;
  float scale_log2;
  hipStream_t stream;
};

hipError_t launch_shared_prefix(const SharedPrefixArgs& a);
hipError_t launch_prefill(const PrefillArgs& a);
hipError_t launch_mixed(const MixedArgs& a);
// the decode merge alone (after launch_mixed wrote the split partials)
hipError_t launch_decode_merge(const DecodeArgs& a);
hipError_t launch_append(const AppendArgs& a);
hipError_t launch_cow(const CowArgs& a);
hipError_t launch_hbm_probe(const void* src, size_t bytes, uint32_t* sink, int num_workgroups,
                            hipStream_t stream);
hipError_t launch_mfma_probe(float* sink, int num_workgroups, int iters, hipStream_t stream);

}  // namespace pa
