// Shared-prefix decode for gfx950: the part of a grouped decode that attends to the blocks a
// group of sequences shares.
//
// Forked sequences (parallel samples of one prompt, beams) hold the same physical blocks for
// their common prefix until a write forces a copy (study-docs "PagedAttention & Continuous
// Batching", section "Copy-on-write"; cloudmash "Batching and PagedAttention", section
// "Sharing blocks"; llmdeepdive "7.8", section "Concept", sharing paragraph).  Plain decode
// reads those blocks once per sequence.  Here a group's shared blocks are read once, and all of
// the group's query rows -- (sequence, query head) pairs of one kv head, e.g. 8 beams x 4 heads
// = 32 -- attend to them together.  With 32 rows sharing every key this is a dense
// contraction, so it runs on MFMA (v_mfma_f32_32x32x16_bf16, fp32 accumulate).
//
// Design (ours): one wave per work item (group, row tile of 32 rows, kv head, split of the
// shared keys).  A group's shared blocks are cut into ceil(shared / split_keys) splits as equal
// as whole blocks allow; the host picks split_keys (at most 64 blocks) as large as keeps one
// work item per compute unit.  Keys stream through LDS 32 at a time, double-buffered, with
// buffer-to-LDS loads (16 per tile, always issued, zeros past the split's end) so a counted
// wait keeps the next tile in flight.  Scores are computed transposed (S^T = K Q^T) so each
// lane holds one query row; P is rounded to bf16 for the P.V product, read through the
// transposing LDS load.  The wave writes (max in log2 units, sum, unnormalised accumulator) per
// row to the decode workspace; the split kernel adds the partials of each sequence's own blocks
// and the merge kernel combines them all (log-sum-exp weighting).
#include "launch.hpp"
#include "mfma_tiles.hpp"

namespace pa {

namespace {

constexpr int kSpRows = 32;                   // rows per wave (one MFMA tile)
constexpr int kSpKeys = 32;                   // keys per LDS tile (two 16-token blocks)
constexpr float kSpLazyLog2 = 8.f;

}  // namespace

template <int G, int D>
__global__ __launch_bounds__(kWave) void pa_shared_prefix_kernel(
    float* __restrict__ ws_ml, float* __restrict__ ws_acc, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ k_cache, const bf16_t* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ group_start,
    const int32_t* __restrict__ shared_blocks, const int32_t* __restrict__ seq_lens,
    int num_seqs, int num_kv_heads, int max_blocks_per_seq,
    int row_tiles, int split_keys, int slot_base, int nsplit_max, float scale_log2) {
  using L = KvTile<D>;
  constexpr int kD = D;
  constexpr int kSpChunks = L::kChunks;
  // loads per tile: two blocks of K and V; the counted waits keep one tile's loads in flight
  constexpr int kTileLoads = 2 * 2 * L::kLoadsPerBlock;
  // 2 x 8 KiB each at head_dim 128 (4 KiB at 64, 16 KiB at 256)
  __shared__ uint4 sK0[kSpKeys * kSpChunks], sK1[kSpKeys * kSpChunks];
  __shared__ uint4 sV0[kSpKeys * kSpChunks], sV1[kSpKeys * kSpChunks];

  const int item = blockIdx.x;
  const int kvh = item % num_kv_heads;
  const int tile = (item / num_kv_heads) % row_tiles;
  const int g = item / num_kv_heads / row_tiles;
  const int split = blockIdx.y;
  // bounds are clamped so that malformed group or prefix arguments cannot address memory
  // outside the sequences' rows and slots
  const int g0 = min(max(group_start[g], 0), num_seqs);
  const int ng = min(group_start[g + 1], num_seqs) - g0;
  if (tile * kSpRows >= ng * G) return;
  const int shared_keys =
      min(max(shared_blocks[g0], 0), seq_lens[g0] / kBlock) * kBlock;   // whole blocks only
  // ns = ceil(shared_keys / split_keys) splits, as the merge counts them, each of whole blocks
  // and as equal as blocks allow: floor or ceil of nb / ns blocks, so none is empty and none
  // is longer than split_keys
  const int ns = (shared_keys + split_keys - 1) / split_keys;
  if (split >= ns) return;
  const int64_t nb = shared_keys / kBlock;
  const int k_begin = static_cast<int>(split * nb / ns) * kBlock;
  const int k_end = static_cast<int>((split + 1) * nb / ns) * kBlock;
  const int num_tiles = (k_end - k_begin + kSpKeys - 1) / kSpKeys;
  // the shared blocks have the same ids in every member's table: read the first member's
  const int32_t* table = block_tables + static_cast<size_t>(g0) * max_blocks_per_seq;
  const size_t slab = static_cast<size_t>(kBlock) * kD;

  const int lane = threadIdx.x;
  const int half = lane / 32;
  const int col = lane % 32;
  const int r = tile * kSpRows + col;
  const int member = r / G;
  const int head = r % G;
  const bool row_valid = member < ng;
  const int seq = g0 + min(member, ng - 1);
  const int Hq = num_kv_heads * G;

  // The split's block ids, one per lane (split_keys <= 64 blocks), read once up front so the
  // tile loop never waits on a table read.
  const int kb0 = k_begin / kBlock;
  const int nb_split = (k_end - k_begin + kBlock - 1) / kBlock;
  const int my_block = lane < nb_split ? table[kb0 + lane] : 0;

  uint4 qreg[kD / 16];
  {
    const bf16_t* qp = q + (static_cast<size_t>(seq) * Hq + kvh * G + head) * kD + half * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qreg[ks] = load16(qp + ks * 16);
  }
  // q and the block ids arrive before any tile load is issued: from here on the only
  // vector-memory loads in flight are the tiles', which the loop counts itself
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // Tile t holds keys k_begin + 32t .. +31: two blocks.  Each block's descriptors cover only
  // its keys below k_end, so keys past the split's end arrive as zeros; all kTileLoads loads
  // are always issued.  In load j of block bi lane l writes LDS row 16 bi + kKeysPerLoad j +
  // l / kChunks, chunk l % kChunks.
  auto load_tile = [&](int t, const uint4* kdst, const uint4* vdst) {
#pragma unroll
    for (int bi = 0; bi < 2; ++bi) {
      const int lblk = t * 2 + bi;                               // block within the split
      // uniform by construction; readfirstlane keeps the clamp off the vector unit so the
      // descriptors stay in scalar registers
      const int rows = wave_uniform(max(0, min(kBlock, k_end - k_begin - lblk * kBlock)));
      const int phys = rows > 0 ? __builtin_amdgcn_readlane(my_block, lblk) : 0;
      const size_t off = (static_cast<size_t>(phys) * num_kv_heads + kvh) * slab;
      const __amdgpu_buffer_rsrc_t krs = buffer_rsrc(k_cache + off, rows * L::kRowBytes);
      const __amdgpu_buffer_rsrc_t vrs = buffer_rsrc(v_cache + off, rows * L::kRowBytes);
#pragma unroll
      for (int j = 0; j < L::kLoadsPerBlock; ++j) {
        const int slot = L::kKeysPerLoad * j + lane / kSpChunks;
        const int key = bi * kBlock + slot;
        const int pchunk = lane % kSpChunks;
        const int row0 = bi * kBlock + L::kKeysPerLoad * j;
        buffer_to_lds16_untracked(krs, lds_addr(kdst + row0 * kSpChunks),
                                  slot * L::kRowBytes + L::kswz(key, pchunk) * 16);
        buffer_to_lds16_untracked(vrs, lds_addr(vdst + row0 * kSpChunks),
                                  slot * L::kRowBytes + L::vswz(key, pchunk) * 16);
      }
    }
  };

  f32x16_t oacc[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
  float m_run = kNegInf;     // raw-score units
  float l_run = 0.f;
  const float lazy_raw = kSpLazyLog2 / scale_log2;
  const int g16 = lane / 16;
  const int jj = lane % 16;

  auto compute = [&](int t, const uint4* kbuf, const uint4* vbuf) {
    // S^T = K Q^T for 32 keys
    f32x16_t sacc;
#pragma unroll
    for (int v = 0; v < 16; ++v) sacc[v] = 0.f;
    {
      const int key = col;
      uint4 a[kD / 16];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks)
        a[ks] = kbuf[key * kSpChunks + L::kswz(key, ks * 2 + half)];
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks)
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[ks]), as_bf16x8(qreg[ks]),
                                                       sacc, 0, 0, 0);
    }
    // keys past the split's end (zero rows) take no weight
    const int key_base = k_begin + t * kSpKeys;
    if (key_base + kSpKeys > k_end) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = key_base + (v / 4) * 8 + half * 4 + (v % 4);
        sacc[v] = key < k_end ? sacc[v] : kNegInf;
      }
    }
    float mx = sacc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = fmaxf(mx, sacc[v]);
    mx = max_with_other_half(mx);
    if (__builtin_amdgcn_ballot_w64(mx > m_run + lazy_raw) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = fast_exp2((m_run - m_new) * scale_log2);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;
    }
    const float mc = m_run * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float p = fast_exp2(fmaf(sacc[v], scale_log2, -mc));
      sacc[v] = p;
      psum += p;
    }
    l_run += psum;
    // P^T operand for k-step s (keys 16s + {0..3, 8..11} + 4*half): the lane's scores 8s..8s+7
    uint4 pT[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int o = s * 8;
      pT[s] = make_uint4(pack_bf16x2(sacc[o + 0], sacc[o + 1]), pack_bf16x2(sacc[o + 2], sacc[o + 3]),
                         pack_bf16x2(sacc[o + 4], sacc[o + 5]), pack_bf16x2(sacc[o + 6], sacc[o + 7]));
    }
    // O^T += V^T P^T; the A operand is two transposing reads (keys +0..3 and +8..11)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      uint4 a[kD / 32];
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt) {
        const int unit = dt * 8 + (g16 % 2) * 4 + (jj % 4);
        uint2 part[2];
#pragma unroll
        for (int sub = 0; sub < 2; ++sub) {
          const int key = 16 * s + 8 * sub + 4 * half + jj / 4;
          const char* rowp = reinterpret_cast<const char*>(vbuf + key * kSpChunks);
          part[sub] = lds_read_tr16(rowp + L::vswz(key, unit >> 1) * 16 + (unit & 1) * 8);
        }
        a[dt] = make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
      }
#pragma unroll
      for (int dt = 0; dt < kD / 32; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[dt]), as_bf16x8(pT[s]),
                                                           oacc[dt], 0, 0, 0);
    }
  };

  // Double buffer: tile t in buffer t % 2.  After tile t is consumed, tile t+2 is requested
  // into its buffer; the counted wait (kTileLoads loads per tile) lets exactly that request
  // stay in flight, and the LDS wait before a reload makes the tile's reads complete first.
  load_tile(0, sK0, sV0);
  load_tile(1, sK1, sV1);
  wait_vmcnt_fence<kTileLoads>();
  for (int t = 0; t < num_tiles; t += 2) {
    compute(t, sK0, sV0);
    lgkm_fence();
    load_tile(t + 2, sK0, sV0);
    wait_vmcnt_fence<kTileLoads>();
    if (t + 1 >= num_tiles) break;
    compute(t + 1, sK1, sV1);
    lgkm_fence();
    load_tile(t + 3, sK1, sV1);
    wait_vmcnt_fence<kTileLoads>();
  }
  wait_vmcnt_fence<0>();     // no load may still be writing LDS when the wave ends

  const float l_tot = add_other_half(l_run);
  if (row_valid) {
    const size_t row = static_cast<size_t>(seq) * Hq + kvh * G + head;
    const size_t slot = row * nsplit_max + (slot_base - ns + split);
    if (half == 0) {
      ws_ml[slot * 2 + 0] = m_run * scale_log2;
      ws_ml[slot * 2 + 1] = l_tot;
    }
    float* ap = ws_acc + slot * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + half * 4;
        *reinterpret_cast<float4*>(ap + d) =
            make_float4(oacc[dt][g4 * 4 + 0], oacc[dt][g4 * 4 + 1], oacc[dt][g4 * 4 + 2],
                        oacc[dt][g4 * 4 + 3]);
      }
  }
}

template <int G, int D>
static hipError_t launch_shared_gd(const SharedPrefixArgs& a) {
  const dim3 grid(a.num_groups * a.row_tiles * a.num_kv_heads, a.nsplit_shared);
  hipLaunchKernelGGL((pa_shared_prefix_kernel<G, D>), grid, dim3(kWave), 0, a.stream, a.ws_ml,
                     a.ws_acc, static_cast<const bf16_t*>(a.q),
                     static_cast<const bf16_t*>(a.k_cache), static_cast<const bf16_t*>(a.v_cache),
                     a.block_tables, a.group_start, a.shared_blocks, a.seq_lens, a.num_seqs,
                     a.num_kv_heads,
                     a.max_blocks_per_seq, a.row_tiles, a.split_keys, a.slot_base, a.nsplit_max,
                     a.scale_log2);
  return hipGetLastError();
}

template <int G>
static hipError_t launch_shared_g(const SharedPrefixArgs& a) {
  switch (a.head_dim) {
    case 64: return launch_shared_gd<G, 64>(a);
    case 128: return launch_shared_gd<G, 128>(a);
    case 256: return launch_shared_gd<G, 256>(a);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_shared_prefix(const SharedPrefixArgs& a) {
  switch (a.num_q_heads / a.num_kv_heads) {
    case 1: return launch_shared_g<1>(a);
    case 2: return launch_shared_g<2>(a);
    case 4: return launch_shared_g<4>(a);
    case 8: return launch_shared_g<8>(a);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
