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
// 256 rows at head_dim 64 and 128, 4 waves and 128 rows at 256; the 4-stage K/V ring in LDS).  Two work queues, each an atomic counter in the workspace that the
// append launch before this one zeroes:
//   * prefill items (chunk, row tile, kv head), longest chunk first (ranked in LDS from
//     seq_lens, as in the prefill kernel);
//   * decode items (sequence, split, kv head), only the splits that exist: every workgroup
//     builds the prefix sum of each sequence's split count in LDS and finds an item's sequence
//     by binary search.
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
// Blocks a decode wave loads together.  The prefill path fixes the register budget (256), so
// deeper batches than the standalone decode's would cost no occupancy, but measured on the
// mixed iteration they were slower (8 and 12 blocks against 4): at two waves per SIMD a wave
// waits for its whole batch before any math, so a deeper batch only lengthens that wait.
constexpr int kMixedDecodeBatch = 0;      // the standalone decode's 64 tokens

}  // namespace

template <int G, int D>
__global__ __launch_bounds__(PfShape<D>::kThreads, 1) void pa_mixed_kernel(
    bf16_t* __restrict__ chunk_out, const bf16_t* __restrict__ chunk_q,
    const int32_t* __restrict__ chunk_tables, const int32_t* __restrict__ chunk_seq_lens,
    const int32_t* __restrict__ query_start_loc, int num_chunks, int chunk_max_blocks,
    bf16_t* __restrict__ dec_out, const bf16_t* __restrict__ dec_q,
    const int32_t* __restrict__ dec_tables, const int32_t* __restrict__ dec_seq_lens,
    int num_seqs, int dec_max_blocks, int bps, int nsplit_max, float* __restrict__ ws_ml,
    float* __restrict__ ws_acc, int* __restrict__ queues, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, int num_kv_heads, float scale_log2) {
  // the prefill ring; a decode item uses the same memory for its scores and partial sums (at
  // most 8192 scores, the split planner's cap, and Waves x G x D partial sums: 32 KiB, within
  // the smallest ring)
  using Sh = PfShape<D>;
  constexpr int kThr = Sh::kThreads;
  constexpr int kRing = Sh::kRing;
  static_assert(kThr >= kRankCap && kMixedSeqCap % kThr == 0, "workgroup shape");
  static_assert(8 * kRing * 16 >= 8192 * 4 && 8 * kRing * 16 >= Sh::kWaves * 8 * D * 4,
                "the ring holds a decode item's scores and partial sums");
  __shared__ uint4 ring[8 * kRing];
  __shared__ PrefillRank rk;
  __shared__ int dscan[kMixedSeqCap];
  __shared__ float dred[Sh::kWaves][G];
  __shared__ float dstat_m[G];
  __shared__ float dstat_l[G];
  __shared__ int s_ticket[2];

  const int tid = threadIdx.x;

  // ------------------------------------------------------------ the two work lists
  prefill_rank<G, Sh::kTileRows>(rk, chunk_seq_lens, query_start_loc, num_chunks, num_kv_heads);
  const int total_prefill = num_chunks > 0 ? rk.scan[num_chunks - 1] : 0;
  // splits per sequence, then an inclusive scan over sequences (blocked: each thread scans a
  // run of consecutive sequences, then the run totals are scanned)
  constexpr int kPer = kMixedSeqCap / kThr;
  {
    int run[kPer];
    int acc = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int sidx = tid * kPer + i;
      int n = 0;
      if (sidx < num_seqs) {
        const int nblk = (dec_seq_lens[sidx] + kBlock - 1) / kBlock;
        n = (nblk + bps - 1) / bps;
      }
      acc += n;
      run[i] = acc;
    }
    reinterpret_cast<int*>(ring)[tid] = acc;     // run totals, scanned in place
    __syncthreads();
    int* tot = reinterpret_cast<int*>(ring);
    for (int off = 1; off < kThr; off <<= 1) {
      const int v = tid >= off ? tot[tid - off] : 0;
      __syncthreads();
      tot[tid] += v;
      __syncthreads();
    }
    const int before = tid > 0 ? tot[tid - 1] : 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) dscan[tid * kPer + i] = before + run[i];
    __syncthreads();
  }
  const int total_decode = num_seqs > 0 ? dscan[num_seqs - 1] * num_kv_heads : 0;
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
      const int j = t / num_kv_heads;              // split index over all sequences
      int lo = 0, hi = num_seqs - 1;               // first sequence with dscan > j
      while (lo < hi) {
        const int mid = (lo + hi) / 2;
        if (dscan[mid] > j) hi = mid; else lo = mid + 1;
      }
      const int s = wave_uniform(lo);
      const int split = j - (s > 0 ? dscan[s - 1] : 0);
      const PagedRows<bf16_t, D, kBlock> rows{
          dec_tables + static_cast<size_t>(s) * dec_max_blocks, num_kv_heads, kvh};
      decode_split_item<bf16_t, D, G, kBlock, Sh::kWaves, kMixedDecodeBatch>(
          dec_out, ws_ml, ws_acc, dec_q, k_cache, v_cache, rows, dec_seq_lens[s], nullptr, 0,
          num_kv_heads, SplitPlan::uniform(bps), nsplit_max, scale_log2, s, kvh, split,
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
                     a.num_seqs, a.dec_max_blocks_per_seq, a.bps, a.nsplit_max, a.ws_ml,
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
