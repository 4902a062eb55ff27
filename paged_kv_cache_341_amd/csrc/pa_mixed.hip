// Single-launch mixed batch for gfx950: the prefill chunks and the decode splits of one
// continuous-batching iteration in one persistent kernel.
//
// Continuous batching runs prompt chunks and decode steps of different requests in the same
// iteration, long prompts cut into chunks so they do not stall the decodes (cloudmash
// "Batching and PagedAttention", section "Continuous batching"; llmdeepdive "PagedAttention &
// continuous batching", section "Concept", continuous-batching paragraph).  After the append,
// the chunk attention and the decode attention are independent.  On MI355X they are bound by
// different units: the chunks by the matrix cores, the decodes by HBM.  Run back to back, each
// leaves the other's unit idle; here they share the chip at the same time.
//
// Design (ours): one workgroup per CU in the prefill item's shape for the head dim (8 waves and
// 256 rows at head_dim 64 and 128, 4 waves and 128 rows at 256; the 4-stage K/V ring in LDS).
// Two work queues, each an atomic counter in the workspace that the append launch before this
// one zeroes:
//   * prefill items (chunk, row tile, kv head), longest chunk first (ranked in LDS from
//     seq_lens, as in the prefill kernel);
//   * decode items (split index, sequence, kv head), only the splits that exist, with the
//     standalone decode's split plan (sizes shrinking toward the later splits): every workgroup
//     sorts the sequences by split count in LDS, ties by index so that every workgroup gets the
//     same order, and the sequences that have a split of index j are then a prefix of it; the
//     queue hands out every sequence's first split, then every second split, and so on, the
//     smallest pieces last.
// Workgroups in alternating groups of eight prefer one queue or the other (workgroups reach
// the 8 XCDs round-robin, so each XCD runs both kinds), and take from the other queue once
// their own is empty; a workgroup leaves when both are.  Decode splits with more than one
// split per sequence write (max, sum, acc) partials that the merge launch after this one
// combines; single-split sequences are written directly.
#include "decode_item.hpp"
#include "launch.hpp"
#include "prefill_item.hpp"

namespace pa {

namespace {

constexpr int kMixedSeqCap = 2048;        // decode sequences enumerated in LDS
constexpr int kMixedLevels = 2048;        // split counts 0 .. 2047 (nsplit_max < 2048)
// Blocks a decode wave loads together.  The prefill path fixes the register budget (256), so
// deeper batches than the standalone decode's would cost no occupancy, but measured on the
// mixed iteration they were slower (8 and 12 blocks against 4): at two waves per SIMD a wave
// waits for its whole batch before any math, so a deeper batch only lengthens that wait.
constexpr int kMixedDecodeBatch = 0;      // the standalone decode's 64 tokens

// Inclusive prefix sums (Suffix: suffix sums) of a[0 .. kN) in LDS, by all kThr threads of the
// workgroup: each thread scans a run of kN / kThr consecutive entries, the run totals are
// scanned in `tot` (kThr ints of LDS), and each run adds what precedes it.
template <int kThr, int kN, bool Suffix>
__device__ __forceinline__ void block_scan(int* a, int* tot) {
  static_assert(kN % kThr == 0, "runs of equal length");
  constexpr int kPer = kN / kThr;
  const int tid = threadIdx.x;
  auto at = [&](int i) -> int& { return a[Suffix ? kN - 1 - i : i]; };
  int run[kPer];
  int acc = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    acc += at(tid * kPer + i);
    run[i] = acc;
  }
  tot[tid] = acc;
  __syncthreads();
  for (int off = 1; off < kThr; off <<= 1) {
    const int v = tid >= off ? tot[tid - off] : 0;
    __syncthreads();
    tot[tid] += v;
    __syncthreads();
  }
  const int before = tid > 0 ? tot[tid - 1] : 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) at(tid * kPer + i) = before + run[i];
  __syncthreads();
}

}  // namespace

template <int G, int D>
__global__ __launch_bounds__(PfShape<D>::kThreads, 1) void pa_mixed_kernel(
    bf16_t* __restrict__ chunk_out, const bf16_t* __restrict__ chunk_q,
    const int32_t* __restrict__ chunk_tables, const int32_t* __restrict__ chunk_seq_lens,
    const int32_t* __restrict__ query_start_loc, int num_chunks, int chunk_max_blocks,
    bf16_t* __restrict__ dec_out, const bf16_t* __restrict__ dec_q,
    const int32_t* __restrict__ dec_tables, const int32_t* __restrict__ dec_seq_lens,
    int num_seqs, int dec_max_blocks, SplitPlan plan, int nsplit_max, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, int* __restrict__ queues, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, int num_kv_heads, float scale_log2) {
  // the prefill ring; a decode item uses the same memory for its scores and partial sums (at
  // most 8192 scores, the split planner's cap, and Waves x G x D partial sums: 32 KiB, within
  // the smallest ring)
  using Sh = PfShape<D>;
  constexpr int kThr = Sh::kThreads;
  constexpr int kRing = Sh::kRing;
  static_assert(kThr >= kRankCap && kMixedLevels % kThr == 0, "workgroup shape");
  static_assert(8 * kRing * 16 >= 8192 * 4 && 8 * kRing * 16 >= Sh::kWaves * 8 * D * 4,
                "the ring holds a decode item's scores and partial sums");
  __shared__ uint4 ring[8 * kRing];
  __shared__ PrefillRank rk;
  __shared__ int dorder[kMixedSeqCap];           // decode sequences, most splits first
  __shared__ int dlevel[kMixedLevels];           // see the work lists below
  __shared__ float dred[Sh::kWaves][G];
  __shared__ float dstat_m[G];
  __shared__ float dstat_l[G];
  __shared__ int s_ticket[2];

  const int tid = threadIdx.x;

  // ------------------------------------------------------------ the two work lists
  prefill_rank<G, Sh::kTileRows>(rk, chunk_seq_lens, query_start_loc, num_chunks, num_kv_heads);
  const int total_prefill = num_chunks > 0 ? rk.scan[num_chunks - 1] : 0;
  // Decode sequences by split count, most first, ties by sequence index, and per split index j
  // the number of sequences that have a split j.  Every workgroup derives the same order (the
  // queue's tickets name items by their place in it), so it is a full sort of distinct keys,
  // not a counting sort whose ties would land in atomic order.  Split counts are 1 ..
  // nsplit_max < kMixedLevels.
  //   dorder: keys (kMixedLevels - 1 - splits) * kMixedSeqCap + sequence, bitonic-sorted
  //   ascending over the next power of two of num_seqs, then the sequence index alone;
  //   dlevel[n]: the sequences with n splits, then (suffix sum) those with at least n, then
  //   the sequences that have split index j (at least j + 1 splits), and finally their
  //   inclusive prefix over j: the decode items (per kv head) of split indexes 0 .. j.
  int* scan_tmp = reinterpret_cast<int*>(ring);  // kThr ints, free until the first item
  int padded = 1;
  while (padded < num_seqs) padded <<= 1;
  for (int i = tid; i < kMixedLevels; i += kThr) dlevel[i] = 0;
  for (int i = tid; i < padded; i += kThr) {
    int key = 0x7fffffff;                          // padding sorts last
    if (i < num_seqs) {
      const int n = min(plan.count((dec_seq_lens[i] + kBlock - 1) / kBlock), nsplit_max);
      key = (kMixedLevels - 1 - n) * kMixedSeqCap + i;
    }
    dorder[i] = key;
  }
  __syncthreads();
  for (int sidx = tid; sidx < num_seqs; sidx += kThr)
    atomicAdd(&dlevel[kMixedLevels - 1 - dorder[sidx] / kMixedSeqCap], 1);
  for (int k = 2; k <= padded; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      __syncthreads();
      for (int i = tid; i < padded; i += kThr) {
        const int ixj = i ^ j;
        if (ixj > i) {
          const int a = dorder[i], b = dorder[ixj];
          if ((a > b) == ((i & k) == 0)) {
            dorder[i] = b;
            dorder[ixj] = a;
          }
        }
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < num_seqs; i += kThr) dorder[i] %= kMixedSeqCap;
  block_scan<kThr, kMixedLevels, true>(dlevel, scan_tmp);
  {
    // split index j exists for the sequences with at least j + 1 splits (j + 1 <= nsplit_max)
    int has[kMixedLevels / kThr];
#pragma unroll
    for (int i = 0; i < kMixedLevels / kThr; ++i) {
      const int j = tid + i * kThr;
      has[i] = j < nsplit_max ? dlevel[j + 1] : 0;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kMixedLevels / kThr; ++i) dlevel[tid + i * kThr] = has[i];
    __syncthreads();
  }
  block_scan<kThr, kMixedLevels, false>(dlevel, scan_tmp);
  const int total_decode =
      num_seqs > 0 && nsplit_max > 0 ? dlevel[nsplit_max - 1] * num_kv_heads : 0;
  const int totals[2] = {total_prefill, total_decode};

  // alternating groups of eight workgroups prefer prefill (0) or decode (1)
  const int prefer = (blockIdx.x / 8) % 2;
  for (;;) {
    if (tid == 0) {
      int which = -1, t = 0;
      for (int attempt = 0; attempt < 2 && which < 0; ++attempt) {
        const int qi = attempt == 0 ? prefer : 1 - prefer;
        if (totals[qi] == 0) continue;
        const int v = __hip_atomic_fetch_add(&queues[qi], 1, __ATOMIC_RELAXED,
                                             __HIP_MEMORY_SCOPE_AGENT);
        if (v < totals[qi]) {
          which = qi;
          t = v;
        }
      }
      s_ticket[0] = which;
      s_ticket[1] = t;
    }
    __syncthreads();
    const int which = wave_uniform(s_ticket[0]);
    const int t = wave_uniform(s_ticket[1]);
    __syncthreads();                               // s_ticket is rewritten next round
    if (which < 0) break;                          // both queues are empty
    if (which == 0) {
      int c, tile, kvh;
      if (prefill_locate<G, Sh::kTileRows>(rk, t, query_start_loc, num_chunks, num_kv_heads, c,
                                           tile, kvh))
        prefill_item<G, D>(chunk_out, chunk_q, k_cache, v_cache, chunk_tables, chunk_seq_lens,
                        query_start_loc, num_kv_heads, chunk_max_blocks, scale_log2, c, tile,
                        kvh, ring + 0 * kRing, ring + 1 * kRing, ring + 2 * kRing,
                        ring + 3 * kRing, ring + 4 * kRing, ring + 5 * kRing, ring + 6 * kRing,
                        ring + 7 * kRing);
    } else {
      const int kvh = t % num_kv_heads;
      const int j = t / num_kv_heads;              // (split index, sequence) pair
      int lo = 0, hi = nsplit_max - 1;             // first split index with dlevel > j
      while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (dlevel[mid] > j) hi = mid; else lo = mid + 1;
      }
      const int split = wave_uniform(lo);
      const int s = wave_uniform(dorder[j - (split > 0 ? dlevel[split - 1] : 0)]);
      const PagedRows<bf16_t, D, kBlock> rows{
          dec_tables + static_cast<size_t>(s) * dec_max_blocks, num_kv_heads, kvh};
      decode_split_item<bf16_t, D, G, kBlock, Sh::kWaves, kMixedDecodeBatch>(
          dec_out, ws_ml, ws_acc, dec_q, k_cache, v_cache, rows, dec_seq_lens[s], nullptr, 0,
          num_kv_heads, plan, nsplit_max, scale_log2, s, kvh, split,
          reinterpret_cast<float*>(ring), dred, dstat_m, dstat_l);
    }
    __syncthreads();                               // the ring is reused by the next item
  }
}

template <int G, int D>
static hipError_t launch_mixed_gd(const MixedArgs& a) {
  hipLaunchKernelGGL((pa_mixed_kernel<G, D>), dim3(a.num_workgroups), dim3(PfShape<D>::kThreads),
                     0, a.stream,
                     static_cast<bf16_t*>(a.chunk_out), static_cast<const bf16_t*>(a.chunk_q),
                     a.chunk_tables, a.chunk_seq_lens, a.query_start_loc, a.num_chunks,
                     a.chunk_max_blocks_per_seq, static_cast<bf16_t*>(a.dec_out),
                     static_cast<const bf16_t*>(a.dec_q), a.dec_tables, a.dec_seq_lens,
                     a.num_seqs, a.dec_max_blocks_per_seq, a.plan, a.nsplit_max, a.ws_ml,
                     a.ws_acc, a.queues, static_cast<const bf16_t*>(a.k_cache),
                     static_cast<const bf16_t*>(a.v_cache), a.num_kv_heads, a.scale_log2);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_mixed_g(const MixedArgs& a) {
  switch (a.head_dim) {
    case 64: return launch_mixed_gd<G, 64>(a);
    case 128: return launch_mixed_gd<G, 128>(a);
    case 256: return launch_mixed_gd<G, 256>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_mixed(const MixedArgs& a) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_mixed_g<1>(a);
    case 2: return launch_mixed_g<2>(a);
    case 4: return launch_mixed_g<4>(a);
    case 8: return launch_mixed_g<8>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
