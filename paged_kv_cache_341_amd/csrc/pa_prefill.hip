// Chunked-prefill attention over a paged prefix, for gfx950 matrix cores.
//
// Operation: chunk c holds the last n rows of a sequence of seq_lens[c] tokens (the chunk was
// appended before this call); row i sits at position P + i, P = seq_lens[c] - n, and attends to
// keys 0 .. P + i, all gathered through the chunk's block table (cloudmash "Batching and
// PagedAttention", sections "Continuous batching" (chunked prefill) and "PagedAttention"
// step 4; study-docs "PagedAttention & Continuous Batching", section "Block tables").
//
// This is a dense contraction, so it runs on MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
// Design (ours):
//   * A work item is (chunk, row tile, kv head).  Rows of a tile are (token, query head) pairs
//     with the G heads of one kv head innermost, so the G heads share every K/V tile.  A
//     workgroup owns 256 rows: 8 waves x 32 rows, one workgroup per CU (two waves per SIMD).
//     That is the shape for head_dim 128 described below, and for head_dim 64 with half-width
//     tiles; at head_dim 256 a workgroup owns 128 rows (4 waves, one per SIMD, whose
//     accumulators and Q operand need more than half a SIMD's registers) and tiles hold 32
//     keys (PfShape in prefill_item.hpp).
//   * Items are dealt longest chunk first (ranked inside the kernel from seq_lens, no host
//     read-back), last row tile first within a chunk, kv head fastest.  Workgroups reach the 8
//     XCDs round-robin in launch order, so with 8 kv heads each XCD serves one head, and the
//     row tiles of one (chunk, head) read the same prefix through the same L2.
//   * Keys go through LDS 64 at a time (four 16-token blocks) in a 4-stage ring: tile t+3 is
//     requested while tile t is computed.  Every wave moves one 16-token block of K (waves
//     0-3) or V (waves 4-7) per tile with four 1 KiB buffer-to-LDS loads whose descriptor
//     covers only the block's valid rows: rows past the sequence end (and blocks past it)
//     arrive as zeros, and every wave issues the same number of loads, so a counted wait
//     (vmcnt) keeps the newest tile in flight across the barrier.  Lanes are permuted so rows
//     land XOR-swizzled.  K and V stay row-major ([key][head_dim], as in the pool); the P.V
//     operand, which needs four consecutive keys of one head-dim column per lane, is read with
//     the gfx950 transposing LDS load (ds_read_b64_tr_b16: in each 16-lane group, lane i
//     receives element i%4 of the 8-byte reads of lanes i/4, 4+i/4, 8+i/4, 12+i/4).
//   * Scores are computed transposed, S^T = K Q^T, so a lane holds one query row: the running
//     max / sum and the rescale of the output accumulator are per-lane scalars, and the
//     probabilities are already laid out as the B operand of O^T = V^T P^T.  P is rounded to
//     bf16 for that product; everything else stays fp32.  The scores of tile t+1 are issued to
//     the matrix cores while the exponentials of tile t run on the vector ALUs.  The running
//     max is raised only when a row's new maximum exceeds it by more than 2^8 in probability
//     (probabilities then stay below 256), so most tiles skip the accumulator rescale.
//   * Masking is by selection (-inf scores), applied only to tiles that reach past a row's
//     position.
#include "launch.hpp"
#include "prefill_item.hpp"

namespace pa {

template <int G, int D>
__global__ __launch_bounds__(PfShape<D>::kThreads, 1) void pa_prefill_kernel(
    bf16_t* __restrict__ out, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ query_start_loc,
    int num_chunks, int num_kv_heads, int max_blocks_per_seq, int tiles_max, float scale_log2) {
  // A 4-stage ring of K and V tiles, as distinct arrays (128 KiB; 64 KiB at head_dim 64).  The
  // loop is unrolled by four so every access names its stage at compile time, which lets the
  // compiler see that the loads into one stage cannot alias the reads of another.
  using Sh = PfShape<D>;
  static_assert(Sh::kThreads >= kRankCap, "the in-kernel ranking gives one chunk per thread");
  __shared__ uint4 sK0[Sh::kRing], sK1[Sh::kRing], sK2[Sh::kRing], sK3[Sh::kRing];
  __shared__ uint4 sV0[Sh::kRing], sV1[Sh::kRing], sV2[Sh::kRing], sV3[Sh::kRing];
  __shared__ PrefillRank rk;

  const int w = blockIdx.x;
  int c, tile, kvh;
  if (num_chunks <= kRankCap) {
    prefill_rank<G, Sh::kTileRows>(rk, seq_lens, query_start_loc, num_chunks, num_kv_heads);
    if (!prefill_locate<G, Sh::kTileRows>(rk, w, query_start_loc, num_chunks, num_kv_heads, c,
                                          tile, kvh))
      return;                                            // past the last item
  } else {
    c = w / (tiles_max * num_kv_heads);
    const int rem = w % (tiles_max * num_kv_heads);
    tile = rem / num_kv_heads;
    kvh = rem % num_kv_heads;
  }
  prefill_item<G, D>(out, q, k_cache, v_cache, block_tables, seq_lens, query_start_loc,
                  num_kv_heads, max_blocks_per_seq, scale_log2, c, tile, kvh, sK0, sK1, sK2, sK3,
                  sV0, sV1, sV2, sV3);
}

template <int G, int D>
static hipError_t launch_prefill_gd(const PrefillArgs& a) {
  using Sh = PfShape<D>;
  const int tiles_max = (a.max_q_len * G + Sh::kTileRows - 1) / Sh::kTileRows;
  const int64_t items = static_cast<int64_t>(a.num_chunks) * tiles_max * a.num_kv_heads;
  hipLaunchKernelGGL((pa_prefill_kernel<G, D>), dim3(static_cast<unsigned>(items)),
                     dim3(Sh::kThreads),
                     0, a.stream, static_cast<bf16_t*>(a.out), static_cast<const bf16_t*>(a.q),
                     static_cast<const bf16_t*>(a.k_cache), static_cast<const bf16_t*>(a.v_cache),
                     a.block_tables, a.seq_lens, a.query_start_loc, a.num_chunks,
                     a.num_kv_heads, a.max_blocks_per_seq, tiles_max, a.scale_log2);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_prefill_g(const PrefillArgs& a) {
  switch (a.head_dim) {
    case 64: return launch_prefill_gd<G, 64>(a);
    case 128: return launch_prefill_gd<G, 128>(a);
    case 256: return launch_prefill_gd<G, 256>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(const PrefillArgs& a) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_prefill_g<1>(a);
    case 2: return launch_prefill_g<2>(a);
    case 4: return launch_prefill_g<4>(a);
    case 8: return launch_prefill_g<8>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
