// Paged decode attention for gfx950.
//
// Operation: one query token per sequence attends to all of that sequence's cached tokens,
// which are gathered through its block table from blocks (16 tokens unless the caller picks
// another size) anywhere in the pool
// (cloudmash "Batching and PagedAttention", section "PagedAttention", step 4; study-docs
// "PagedAttention & Continuous Batching", section "Block tables").  Query head h reads kv head
// h / G, G = Hq / Hkv, so the G query heads of one kv head share every K/V byte read.
//
// Work split (our design, not from the pages): one workgroup of 4 waves per
// (sequence, kv head, split), a split being a run of consecutive logical blocks (its length
// set by the host's split plan, which may shrink toward the later splits).  Inside a split:
//   phase 1  each wave takes every 4th unit of the split (a block of 8 or 16 tokens, a
//            16-token run of a larger block, or 16 tokens of smaller blocks), reads its K rows,
//            computes the G scores of every token with lanes split over the head dimension
//            (DPP sums), and parks them in LDS;
//   phase 2  exact softmax statistics of the split: max and sum of exp2 per query head;
//   phase 3  each wave reads the V rows of the same units and accumulates p * V in fp32,
//            lanes split over the head dimension again; waves are summed through LDS.
// Wave priorities: on a CU the oldest waves win instruction issue, so workgroups dispatched
// late (onto slots freed by finished splits) were starved by older ones and ended the kernel
// late.  Each split therefore runs its K phase at a higher wave priority than its V phase, so
// the splits that have made the least progress issue first, and the splits dispatched last
// (the second half of the split index range) sit one band above the rest.
// A split with the whole sequence writes the normalised output; otherwise it writes
// (max, sum, unnormalised acc) and a merge kernel combines the splits in split order
// (log-sum-exp weighting), so results do not depend on scheduling.
// Only the last block of a sequence can be partly filled; its unfilled slots are masked by
// selection (score -inf, V treated as 0), never by multiplying, so garbage there is harmless.
#include "decode_item.hpp"
#include "launch.hpp"

namespace pa {

// U: tokens per unit of the split walk (the pool's block size when BT == U); BT: tokens per
// pool block (BT < U: blocks smaller than a unit, looked up per token; BT > U: blocks holding
// several units); Contig: no table, the cache is [num_seqs][num_kv_heads][capacity][D].
template <typename T, int D, int G, int U, int BT, bool Contig>
__global__ __launch_bounds__(kDecodeThreads) void pa_decode_split_kernel(
    T* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ skip_blocks, int slot_base, int num_kv_heads,
    int max_blocks_per_seq, int capacity, SplitPlan plan, int nsplit_max, float scale_log2) {
  extern __shared__ float smem[];
  __shared__ float red[kDecodeWaves][G];
  __shared__ float stat_m[G];
  __shared__ float stat_l[G];
  // grid.x runs over (sequence, kv head) and grid.y over splits, so consecutive workgroups
  // belong to different kv heads.  Workgroups are dealt to the 8 XCDs round-robin in launch
  // order; with this order each XCD gets an even share of every split index (instead of one
  // XCD holding every sequence's first split), and the beams that share a block read it
  // through the same XCD's L2.
  // The splits dispatched last are the second half of the split-index range (grid.y): they
  // take the higher of the two priority bands (see decode_split_item).
  const int s = static_cast<int>(blockIdx.x) / num_kv_heads;
  const int kvh = static_cast<int>(blockIdx.x) % num_kv_heads;
  const int L = seq_lens[s];
  const bool late = blockIdx.y * 2 >= gridDim.y;
  if constexpr (Contig) {
    const ContiguousRows<T, D, U> rows{(static_cast<size_t>(s) * num_kv_heads + kvh) *
                                       static_cast<size_t>(capacity) * D};
    decode_split_item<T, D, G, U, kDecodeWaves, 0, true>(
        out, ws_ml, ws_acc, q, k_cache, v_cache, rows, L, skip_blocks, slot_base, num_kv_heads,
        plan, nsplit_max, scale_log2, s, kvh, static_cast<int>(blockIdx.y), smem, red, stat_m,
        stat_l, late);
  } else if constexpr (BT == U) {
    const PagedRows<T, D, U> rows{block_tables + static_cast<size_t>(s) * max_blocks_per_seq,
                                  num_kv_heads, kvh};
    decode_split_item<T, D, G, U, kDecodeWaves, 0, true>(
        out, ws_ml, ws_acc, q, k_cache, v_cache, rows, L, skip_blocks, slot_base, num_kv_heads,
        plan, nsplit_max, scale_log2, s, kvh, static_cast<int>(blockIdx.y), smem, red, stat_m,
        stat_l, late);
  } else if constexpr (BT > U) {
    const PagedLargeRows<T, D, U, BT> rows{
        block_tables + static_cast<size_t>(s) * max_blocks_per_seq, num_kv_heads, kvh};
    decode_split_item<T, D, G, U, kDecodeWaves, 0, true>(
        out, ws_ml, ws_acc, q, k_cache, v_cache, rows, L, skip_blocks, slot_base, num_kv_heads,
        plan, nsplit_max, scale_log2, s, kvh, static_cast<int>(blockIdx.y), smem, red, stat_m,
        stat_l, late);
  } else {
    const PagedSmallRows<T, D, U, BT> rows{
        block_tables + static_cast<size_t>(s) * max_blocks_per_seq, num_kv_heads, kvh, L};
    decode_split_item<T, D, G, U, kDecodeWaves, 0, true>(
        out, ws_ml, ws_acc, q, k_cache, v_cache, rows, L, skip_blocks, slot_base, num_kv_heads,
        plan, nsplit_max, scale_log2, s, kvh, static_cast<int>(blockIdx.y), smem, red, stat_m,
        stat_l, late);
  }
}

// Combine the splits of one (sequence, query head) row; one wave per row.  Lanes first read
// the per-split (max, sum) pairs in parallel, so the split count costs one round trip rather
// than a chain of dependent loads; then each lane owns D/64 output elements and sums the
// splits' weighted partial numerators in split order (the same order on every run).
constexpr int kMergeWaves = 4;

template <typename T, int D, int B>
__global__ __launch_bounds__(kMergeWaves * kWave) void pa_decode_merge_kernel(
    T* __restrict__ out, const float* __restrict__ ws_ml, const float* __restrict__ ws_acc,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ skip_blocks,
    int slot_base, int shared_split_keys, int num_rows, int num_q_heads, SplitPlan plan,
    int nsplit_max) {
  constexpr int kPer = D / kWave;
  constexpr int kFast = 16;
  const int row = blockIdx.x * kMergeWaves + static_cast<int>(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  if (row >= num_rows) return;
  const int s = row / num_q_heads;

  if (skip_blocks == nullptr && slot_base == 0 && nsplit_max <= kFast) {
    // Plain decode with at most kFast split slots per row: the row's split count follows from
    // the sequence length, then the statistics and partials of exactly those splits are
    // requested together (one round trip).  Reading every slot of the row with the length
    // instead saves that dependent load but fetches the unused slots too; with the shrinking
    // split plans (11 slots for 4096-token rows, 5 used on average) that cost more.
    const float* ml = ws_ml + static_cast<size_t>(row) * nsplit_max * 2;
    const float* acc = ws_acc + static_cast<size_t>(row) * nsplit_max * D;
    const int L = seq_lens[s];
    const int nsplit = plan.count((L + B - 1) / B);
    if (nsplit <= 1) return;                      // written directly by the split kernel
    float a[kFast][kPer];
#pragma unroll
    for (int u = 0; u < kFast; ++u)
      if (u < nsplit)
#pragma unroll
        for (int e = 0; e < kPer; ++e) a[u][e] = acc[static_cast<size_t>(u) * D + lane + e * kWave];
    const float mraw = lane < nsplit ? ml[2 * lane] : 0.f;
    const float lraw = lane < nsplit ? ml[2 * lane + 1] : 0.f;
    const float mi = lane < nsplit ? mraw : kNegInf;
    const float li = lane < nsplit ? lraw : 0.f;
    const float Mf = group_max<kWave>(mi);
    const float w = lane < nsplit ? exp2f(mi - Mf) : 0.f;
    const float inv = 1.f / group_sum<kWave>(w * li);
    float num[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) num[e] = 0.f;
#pragma unroll
    for (int u = 0; u < kFast; ++u)
      if (u < nsplit) {
        const float wu = u32_as_f32(__builtin_amdgcn_readlane(f32_as_u32(w), u));
#pragma unroll
        for (int e = 0; e < kPer; ++e) num[e] = fmaf(wu, a[u][e], num[e]);
      }
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      store_out(out + static_cast<size_t>(row) * D + lane + e * kWave, num[e] * inv);
    return;
  }

  const int L = seq_lens[s];
  const int nblk = (L + B - 1) / B;
  // partials of this row: the shared-prefix splits end at slot_base, the splits of the rest
  // start there, so they form one range
  const int skip = skip_blocks ? min(max(skip_blocks[s], 0), L / B) : 0;
  const int ns = skip > 0 ? (skip * B + shared_split_keys - 1) / shared_split_keys : 0;
  const int nt = plan.count(nblk - skip);
  if (ns == 0 && nt <= 1) return;                 // written directly by the split kernel
  const int nsplit = ns + nt;
  const float* ml = ws_ml + (static_cast<size_t>(row) * nsplit_max + slot_base - ns) * 2;
  const float* acc = ws_acc + (static_cast<size_t>(row) * nsplit_max + slot_base - ns) * D;

  if (nsplit <= kFast) {
    // Up to kFast splits: the statistics and every partial are requested together, one round
    // trip, and summed in split order as below.
    float a[kFast][kPer];
#pragma unroll
    for (int u = 0; u < kFast; ++u)
      if (u < nsplit)
#pragma unroll
        for (int e = 0; e < kPer; ++e) a[u][e] = acc[static_cast<size_t>(u) * D + lane + e * kWave];
    const float mi = lane < nsplit ? ml[2 * lane] : kNegInf;
    const float li = lane < nsplit ? ml[2 * lane + 1] : 0.f;
    const float Mf = group_max<kWave>(mi);
    const float w = lane < nsplit ? exp2f(mi - Mf) : 0.f;
    const float inv = 1.f / group_sum<kWave>(w * li);
    float num[kPer];
#pragma unroll
    for (int e = 0; e < kPer; ++e) num[e] = 0.f;
#pragma unroll
    for (int u = 0; u < kFast; ++u)
      if (u < nsplit) {
        const float wu = u32_as_f32(__builtin_amdgcn_readlane(f32_as_u32(w), u));
#pragma unroll
        for (int e = 0; e < kPer; ++e) num[e] = fmaf(wu, a[u][e], num[e]);
      }
#pragma unroll
    for (int e = 0; e < kPer; ++e)
      store_out(out + static_cast<size_t>(row) * D + lane + e * kWave, num[e] * inv);
    return;
  }

  float M = kNegInf;
  for (int i = lane; i < nsplit; i += kWave) M = fmaxf(M, ml[2 * i]);
  M = group_max<kWave>(M);
  float den = 0.f;
  for (int i = lane; i < nsplit; i += kWave) den = fmaf(exp2f(ml[2 * i] - M), ml[2 * i + 1], den);
  den = group_sum<kWave>(den);
  const float inv = 1.f / den;

  float num[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) num[e] = 0.f;
  for (int c = 0; c < nsplit; c += kWave) {
    const int i = c + lane;
    const float w = i < nsplit ? exp2f(ml[2 * i] - M) : 0.f;   // this lane's split weight
    const int cnt = min(kWave, nsplit - c);
    int k = 0;
    for (; k + 4 <= cnt; k += 4) {
      float a[4][kPer];
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int e = 0; e < kPer; ++e) a[u][e] = acc[static_cast<size_t>(c + k + u) * D + lane + e * kWave];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float wu = u32_as_f32(__builtin_amdgcn_readlane(f32_as_u32(w), k + u));
#pragma unroll
        for (int e = 0; e < kPer; ++e) num[e] = fmaf(wu, a[u][e], num[e]);
      }
    }
    for (; k < cnt; ++k) {
      const float wk = u32_as_f32(__builtin_amdgcn_readlane(f32_as_u32(w), k));
#pragma unroll
      for (int e = 0; e < kPer; ++e)
        num[e] = fmaf(wk, acc[static_cast<size_t>(c + k) * D + lane + e * kWave], num[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < kPer; ++e) store_out(out + static_cast<size_t>(row) * D + lane + e * kWave, num[e] * inv);
}

template <typename T, int D, int G, int U, int BT, bool Contig>
hipError_t launch_decode_tb(const DecodeArgs& a) {
  const size_t lds = std::max<size_t>(static_cast<size_t>(a.plan.max_units()) * U * G,
                                      static_cast<size_t>(kDecodeWaves) * G * D) * sizeof(float);
  const dim3 grid_split(a.num_seqs * a.num_kv_heads, a.nsplit_tail);
  hipLaunchKernelGGL((pa_decode_split_kernel<T, D, G, U, BT, Contig>), grid_split,
                     dim3(kDecodeThreads), lds, a.stream, static_cast<T*>(a.out), a.ws_ml,
                     a.ws_acc, static_cast<const T*>(a.q), static_cast<const T*>(a.k_cache),
                     static_cast<const T*>(a.v_cache), a.block_tables, a.seq_lens,
                     a.skip_blocks, a.slot_base, a.num_kv_heads, a.max_blocks_per_seq,
                     a.capacity, a.plan, a.nsplit_max, a.scale_log2);
  if (a.nsplit_max > 1) {
    const int rows = a.num_seqs * a.num_kv_heads * G;
    hipLaunchKernelGGL((pa_decode_merge_kernel<T, D, U>),
                       dim3((rows + kMergeWaves - 1) / kMergeWaves), dim3(kMergeWaves * kWave), 0,
                       a.stream, static_cast<T*>(a.out), a.ws_ml, a.ws_acc, a.seq_lens,
                       a.skip_blocks, a.slot_base, a.shared_split_keys, rows,
                       a.num_kv_heads * G, a.plan, a.nsplit_max);
  }
  return hipGetLastError();
}

// The merge for the partials of bf16, 16-token-unit splits written by another kernel.
template <int D>
static hipError_t launch_decode_merge_d(const DecodeArgs& a) {
  const int rows = a.num_seqs * a.num_q_heads;
  hipLaunchKernelGGL((pa_decode_merge_kernel<bf16_t, D, 16>),
                     dim3((rows + kMergeWaves - 1) / kMergeWaves), dim3(kMergeWaves * kWave), 0,
                     a.stream, static_cast<bf16_t*>(a.out), a.ws_ml, a.ws_acc, a.seq_lens,
                     a.skip_blocks, a.slot_base, a.shared_split_keys, rows, a.num_q_heads,
                     a.plan, a.nsplit_max);
  return hipGetLastError();
}

hipError_t launch_decode_merge(const DecodeArgs& a) {
  if (a.nsplit_max <= 1) return hipSuccess;
  switch (a.head_dim) {
    case 64: return launch_decode_merge_d<64>(a);
    case 128: return launch_decode_merge_d<128>(a);
    case 256: return launch_decode_merge_d<256>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a) {
  if (a.contiguous) return launch_decode_tb<T, D, G, 16, 16, true>(a);
  switch (a.block_size) {
    case 1: return launch_decode_tb<T, D, G, 16, 1, false>(a);
    case 4: return launch_decode_tb<T, D, G, 16, 4, false>(a);
    case 8: return launch_decode_tb<T, D, G, 8, 8, false>(a);
    case 16: return launch_decode_tb<T, D, G, 16, 16, false>(a);
    case 32: return launch_decode_tb<T, D, G, 16, 32, false>(a);
    case 64: return launch_decode_tb<T, D, G, 16, 64, false>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D>
hipError_t launch_decode_d(const DecodeArgs& a) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_decode_t<T, D, 1>(a);
    case 2: return launch_decode_t<T, D, 2>(a);
    case 4: return launch_decode_t<T, D, 4>(a);
    case 8: return launch_decode_t<T, D, 8>(a);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_decode_dt(const DecodeArgs& a) {
  switch (a.head_dim) {
    case 64: return launch_decode_d<T, 64>(a);
    case 128: return launch_decode_d<T, 128>(a);
    case 256: return launch_decode_d<T, 256>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a) {
  return a.bf16 ? launch_decode_dt<bf16_t>(a) : launch_decode_dt<float>(a);
}

}  // namespace pa
