// Chunked-prefill work items as device functions (ranking, item lookup, one item), for the
// standalone prefill kernel and the single-launch mixed kernel.  The algorithm is described at
// the top of pa_prefill.hip.
#pragma once

#include "mfma_tiles.hpp"

namespace pa {

namespace {

constexpr int kRowsPerWave = 32;
constexpr int kRankCap = 128;                       // chunks ranked longest-first in-kernel
constexpr float kLazyLog2 = 8.f;                    // rescale only past 2^8 growth

}  // namespace

// The work-item shape for head_dim D.  D 64 and 128: eight waves of 32 rows, 64-key tiles.
// D 256: its fp32 accumulators (128 per lane) and Q operand do not fit two waves per SIMD, so
// four waves of 32 rows (one per SIMD) and 32-key tiles, which keep the 4-stage ring at
// 128 KiB.  In every shape half the waves stage K and half V, one 16-token block each per tile.
template <int D>
struct PfShape : KvTile<D> {
  using L = KvTile<D>;
  static constexpr int kD = D;
  static constexpr int kWaves = D == 256 ? 4 : 8;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int kTileRows = kWaves * kRowsPerWave;
  static constexpr int kKvTile = D == 256 ? 32 : 64;      // keys per LDS tile
  static constexpr int kKeySub = kKvTile / 32;           // 32-key score tiles per LDS tile
  static constexpr int kPvSteps = kKvTile / 16;          // 16-key P.V products per d tile
  static constexpr int kLoads = L::kLoadsPerBlock;       // 1 KiB loads per staged block
  static constexpr int kRing = kKvTile * L::kChunks;     // uint4 per K or V ring stage
  static_assert(kWaves / 2 == kKvTile / kBlock, "one wave stages each K and each V block");
};

// Longest-first order of up to kRankCap chunks, kept in LDS: chunk c's items occupy
// [end[c] - items[c], end[c]) of the item sequence, chunks ranked by length (descending, ties
// by index); within a chunk the last row tile comes first and the kv head varies fastest.
struct PrefillRank {
  int len[kRankCap];
  int scan[kRankCap];
  int end[kRankCap];
  int items[kRankCap];
  int item[2];
};

// Every thread of the workgroup calls this (it synchronises); num_chunks <= kRankCap, and the
// workgroup has at least kRankCap threads.
template <int G, int TileRows>
__device__ __forceinline__ void prefill_rank(PrefillRank& rk, const int32_t* __restrict__ seq_lens,
                                             const int32_t* __restrict__ query_start_loc,
                                             int num_chunks, int num_kv_heads) {
  const int tid = threadIdx.x;
  int my_len = 0, my_items = 0, my_rank = 0;
  if (tid < num_chunks) {
    my_len = seq_lens[tid];
    const int n = query_start_loc[tid + 1] - query_start_loc[tid];
    my_items = (n * G + TileRows - 1) / TileRows * num_kv_heads;
    rk.len[tid] = my_len;
    rk.items[tid] = my_items;
  }
  __syncthreads();
  if (tid < num_chunks) {
    for (int j = 0; j < num_chunks; ++j) {
      const int lj = rk.len[j];
      my_rank += (lj > my_len) || (lj == my_len && j < tid);
    }
    rk.scan[my_rank] = my_items;
  }
  __syncthreads();
  // inclusive scan of the items in rank order
  for (int off = 1; off < kRankCap; off <<= 1) {
    int v = 0;
    if (tid < num_chunks && tid >= off) v = rk.scan[tid - off];
    __syncthreads();
    if (tid < num_chunks) rk.scan[tid] += v;
    __syncthreads();
  }
  if (tid < num_chunks) rk.end[tid] = rk.scan[my_rank];
  __syncthreads();
}

// Item w of the longest-first order as (chunk, row tile, kv head); false past the last item.
// Every thread of the workgroup calls this (it synchronises).
template <int G, int TileRows>
__device__ __forceinline__ bool prefill_locate(PrefillRank& rk, int w,
                                               const int32_t* __restrict__ query_start_loc,
                                               int num_chunks, int num_kv_heads, int& c,
                                               int& tile, int& kvh) {
  const int tid = threadIdx.x;
  if (tid == 0) rk.item[0] = -1;
  __syncthreads();
  if (tid < num_chunks && w >= rk.end[tid] - rk.items[tid] && w < rk.end[tid]) {
    rk.item[0] = tid;
    rk.item[1] = w - (rk.end[tid] - rk.items[tid]);
  }
  __syncthreads();
  c = wave_uniform(rk.item[0]);     // uniform, so table lookups become scalar loads
  const int local = wave_uniform(rk.item[1]);
  __syncthreads();                  // item[] is rewritten by the next call
  if (c < 0) return false;
  const int n = query_start_loc[c + 1] - query_start_loc[c];
  const int tiles = (n * G + TileRows - 1) / TileRows;
  tile = tiles - 1 - local / num_kv_heads;
  kvh = local % num_kv_heads;
  return true;
}

// One work item (chunk c, row tile, kv head) with all PfShape<D>::kThreads threads of the
// workgroup; the eight arrays are the 4-stage K/V ring, each kKvTile x kChunks 16-byte chunks.
template <int G, int D>
__device__ __forceinline__ void prefill_item(
    bf16_t* __restrict__ out, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ query_start_loc,
    int num_kv_heads, int max_blocks_per_seq, float scale_log2, int c, int tile, int kvh,
    uint4* sK0, uint4* sK1, uint4* sK2, uint4* sK3, uint4* sV0, uint4* sV1, uint4* sV2,
    uint4* sV3) {
  using Sh = PfShape<D>;
  constexpr int kD = Sh::kD;
  constexpr int kChunks = Sh::kChunks;
  constexpr int kRowBytes = Sh::kRowBytes;
  constexpr int kKvTile = Sh::kKvTile;
  constexpr int kTokPerTile = Sh::kTileRows / G;
  constexpr int kWaitTile = wait_vmcnt(Sh::kLoads);   // one tile's loads still in flight
  const int tid = threadIdx.x;
  const int q0 = query_start_loc[c];
  const int n = query_start_loc[c + 1] - q0;
  const int t_begin = tile * kTokPerTile;
  if (t_begin >= n) return;
  const int L = seq_lens[c];
  const int prefix = L - n;
  const int nblk = (L + kBlock - 1) / kBlock;
  const int Hq = num_kv_heads * G;
  const int32_t* table = block_tables + static_cast<size_t>(c) * max_blocks_per_seq;
  const size_t slab = static_cast<size_t>(kBlock) * kD;

  const int wave = wave_uniform(tid / kWave);
  const int lane = tid % kWave;
  const int half = lane / 32;        // which 8-wide k slice of an MFMA operand this lane holds
  const int col = lane % 32;         // query row (within the wave) this lane holds

  // rows of this lane and of this wave
  const int r = wave * kRowsPerWave + col;
  const int t_row = t_begin + r / G;
  const bool row_valid = t_row < n;
  const int pos = prefix + min(t_row, n - 1);
  const int t_lo_w = t_begin + (wave * kRowsPerWave) / G;
  const int t_hi_w = min(t_begin + (wave * kRowsPerWave + kRowsPerWave - 1) / G, n - 1);
  const int kv_end_w = prefix + t_hi_w + 1;                  // keys this wave needs
  const int kv_end = prefix + min(t_begin + kTokPerTile, n);  // keys the workgroup needs
  const int num_kv_tiles = (kv_end + kKvTile - 1) / kKvTile;

  // Q^T operand: lane holds row `col`, head-dim slice ks*16 + half*8 .. +8
  uint4 qreg[kD / 16];
  {
    const int t = min(t_row, n - 1);
    const bf16_t* qp =
        q + (static_cast<size_t>(q0 + t) * Hq + kvh * G + (r % G)) * kD + half * 8;
#pragma unroll
    for (int ks = 0; ks < kD / 16; ++ks) qreg[ks] = load16(qp + ks * 16);
  }

  // ------------------------------------------------------------------ tile staging
  // Wave w moves block (w % 4) of a tile, K for w < 4 and V otherwise.  Its descriptor covers
  // exactly the block's valid rows, so rows past the sequence end (and blocks past it, whose
  // table entry is not read) come in as zeros.  In load j lane l writes LDS chunk
  // (16*blk + 4j + l/16, l%16) and so fetches the logical chunk whose swizzled position that is.
  const int stage_blk = wave % (Sh::kWaves / 2);
  const bool stage_v = wave >= Sh::kWaves / 2;
  const bf16_t* stage_pool = stage_v ? v_cache : k_cache;
  auto load_tile = [&](int kt, uint4* kdst, uint4* vdst) {
    // uniform, so the table read is a scalar load
    const int lb = wave_uniform(kt * (kKvTile / kBlock) + stage_blk);
    const int first = lb * kBlock;
    const int rows = max(0, min(kBlock, L - first));
    const int phys = lb < nblk ? wave_uniform(table[lb]) : 0;
    const bf16_t* src = stage_pool + (static_cast<size_t>(phys) * num_kv_heads + kvh) * slab;
    // the descriptor's fields are uniform by construction; saying so keeps it in scalar
    // registers (otherwise the compiler wraps every load in a loop over distinct descriptors)
    const uint64_t sa = reinterpret_cast<uint64_t>(src);
    const uint64_t su =
        (static_cast<uint64_t>(static_cast<uint32_t>(wave_uniform(static_cast<int>(sa >> 32))))
         << 32) |
        static_cast<uint32_t>(wave_uniform(static_cast<int>(sa)));
    __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<bf16_t*>(su), 0, wave_uniform(rows * kRowBytes), kRsrcWord3);
    uint4* dst = (stage_v ? vdst : kdst) + stage_blk * kBlock * kChunks;
#pragma unroll
    for (int j = 0; j < Sh::kLoads; ++j) {
      const int slot = Sh::kKeysPerLoad * j + lane / kChunks;
      const int key = stage_blk * kBlock + slot;
      const int pchunk = lane % kChunks;
      const int lchunk = stage_v ? Sh::vswz(key, pchunk) : Sh::kswz(key, pchunk);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void_t*)(dst + j * kWave), 16,
                                               slot * kRowBytes + lchunk * 16, 0, 0, 0);
    }
  };

  f32x16_t oacc[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
  float m_run = kNegInf;     // raw-score units
  float l_run = 0.f;
  const float lazy_raw = kLazyLog2 / scale_log2;

  // S^T = K Q^T for one 64-key tile.  Operands are read half the head dim at a time, and the
  // two key subtiles' MFMAs alternate so back-to-back MFMAs never depend on each other.
  auto qk = [&](const uint4* kbuf, f32x16_t (&sacc)[Sh::kKeySub]) {
#pragma unroll
    for (int t2 = 0; t2 < Sh::kKeySub; ++t2)
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[t2][v] = 0.f;
#pragma unroll
    for (int kh = 0; kh < kD / 64; ++kh) {
      uint4 a[Sh::kKeySub][4];
#pragma unroll
      for (int t2 = 0; t2 < Sh::kKeySub; ++t2) {
        const int key = t2 * 32 + col;
#pragma unroll
        for (int k4 = 0; k4 < 4; ++k4)
          a[t2][k4] = kbuf[key * kChunks + Sh::kswz(key, (kh * 4 + k4) * 2 + half)];
      }
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
        for (int t2 = 0; t2 < Sh::kKeySub; ++t2)
          sacc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              as_bf16x8(a[t2][k4]), as_bf16x8(qreg[kh * 4 + k4]), sacc[t2], 0, 0, 0);
    }
  };

  // One step of the pipeline, for tile kt whose scores are already in `cur`:
  //   request tile kt+3 into the free stage; issue the QK MFMAs of tile kt+1 into `nxt` while
  //   the softmax of tile kt runs on the vector ALUs; O^T += V(kt)^T P(kt)^T; then wait until
  //   only tile kt+3 is still in flight (tile kt+2 is what the next step reads) and publish.
  // Tile t lives in stage t % 4.  A request past the last tile loads only zeros.
  auto step = [&](int kt, const uint4* knext, const uint4* vcur, uint4* kload, uint4* vload,
                  f32x16_t (&cur)[Sh::kKeySub], f32x16_t (&nxt)[Sh::kKeySub]) {
    load_tile(kt + 3, kload, vload);

    if (kt * kKvTile < kv_end_w) {
      // scores of the next tile first: they depend only on staged K and the resident Q, so the
      // matrix cores work through them while the softmax of tile kt below runs on the vector
      // ALUs (a wave that needs no key of tile kt needs none of tile kt+1 either, and past the
      // last tile the result is simply never used)
      qk(knext, nxt);

      // --------------------------------------------------------------- online softmax (max)
      const bool need_mask = kt * kKvTile + kKvTile - 1 > prefix + t_lo_w;
      if (need_mask) {
#pragma unroll
        for (int t2 = 0; t2 < Sh::kKeySub; ++t2)
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int key = kt * kKvTile + t2 * 32 + (v / 4) * 8 + half * 4 + (v % 4);
            cur[t2][v] = key <= pos ? cur[t2][v] : kNegInf;
          }
      }
      float mx = cur[0][0];
#pragma unroll
      for (int t2 = 0; t2 < Sh::kKeySub; ++t2)
#pragma unroll
        for (int v = 0; v < 16; ++v) mx = fmaxf(mx, cur[t2][v]);
      mx = max_with_other_half(mx);
      // raise the running max only when some row of the wave grew past the lazy margin
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

      // --------------------------------------------------------------- probabilities
      const float mc = m_run * scale_log2;
      float psum = 0.f;
#pragma unroll
      for (int t2 = 0; t2 < Sh::kKeySub; ++t2)
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const float p = fast_exp2(fmaf(cur[t2][v], scale_log2, -mc));
          cur[t2][v] = p;
          psum += p;
        }
      l_run += psum;

      // P^T operand for k-step s: the lane's own scores v = (s%2)*8 .. +8 of key subtile s/2
      uint4 pT[Sh::kPvSteps];
#pragma unroll
      for (int s = 0; s < Sh::kPvSteps; ++s) {
        const f32x16_t& p = cur[s / 2];
        const int o = (s % 2) * 8;
        pT[s] = make_uint4(pack_bf16x2(p[o + 0], p[o + 1]), pack_bf16x2(p[o + 2], p[o + 3]),
                           pack_bf16x2(p[o + 4], p[o + 5]), pack_bf16x2(p[o + 6], p[o + 7]));
      }

      // --------------------------------------------------------------- O^T += V^T P^T
      // k-step s covers keys 16s + {0..3, 8..11} + 4*half for this lane's half (the order the
      // scores sit in); the A operand (d = dt*32 + col, those 8 keys) is two transposing reads,
      // keys +0..3 and +8..11.  Lane l = 16g + j reads key row (.. + j/4), 8-byte unit
      // dt*8 + (g%2)*4 + j%4 of it.
      const int g = lane / 16;
      const int jj = lane % 16;
#pragma unroll
      for (int s = 0; s < Sh::kPvSteps; ++s) {
        uint4 a[kD / 32];
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt) {
          const int unit = dt * 8 + (g % 2) * 4 + (jj % 4);   // 8-byte unit of the d range
          uint2 part[2];
#pragma unroll
          for (int sub = 0; sub < 2; ++sub) {
            const int key = 16 * s + 8 * sub + 4 * half + jj / 4;
            const char* rowp = reinterpret_cast<const char*>(vcur + key * kChunks);
            part[sub] = lds_read_tr16(rowp + Sh::vswz(key, unit >> 1) * 16 + (unit & 1) * 8);
          }
          a[dt] = make_uint4(part[0].x, part[0].y, part[1].x, part[1].y);
        }
#pragma unroll
        for (int dt = 0; dt < kD / 32; ++dt)
          oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a[dt]), as_bf16x8(pT[s]),
                                                             oacc[dt], 0, 0, 0);
      }
    }

    // every wave issued exactly kLoads loads per step: the newest (tile kt+3) may stay in
    // flight, everything older (tile kt+2, read next step) must have landed.  A bare
    // s_barrier, not __syncthreads: its memory fence would wait for the prefetch as well.
    __builtin_amdgcn_s_waitcnt(kWaitTile);
    __builtin_amdgcn_s_barrier();
  };

  // prologue: tiles 0, 1, 2 requested; tiles 0 and 1 landed; scores of tile 0
  load_tile(0, sK0, sV0);
  load_tile(1, sK1, sV1);
  load_tile(2, sK2, sV2);
  __builtin_amdgcn_s_waitcnt(kWaitTile);
  __builtin_amdgcn_s_barrier();
  f32x16_t sa[Sh::kKeySub], sb[Sh::kKeySub];
  qk(sK0, sa);
  for (int kt = 0; kt < num_kv_tiles; kt += 4) {
    step(kt, sK1, sV0, sK3, sV3, sa, sb);
    if (kt + 1 >= num_kv_tiles) break;
    step(kt + 1, sK2, sV1, sK0, sV0, sb, sa);
    if (kt + 2 >= num_kv_tiles) break;
    step(kt + 2, sK3, sV2, sK1, sV1, sa, sb);
    if (kt + 3 >= num_kv_tiles) break;
    step(kt + 3, sK0, sV3, sK2, sV2, sb, sa);
  }
  // no load may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(kWaitVm0);

  // ------------------------------------------------------------------------- write out
  const float l_tot = add_other_half(l_run);
  const float inv = 1.f / l_tot;
  if (row_valid) {
    bf16_t* op = out + (static_cast<size_t>(q0 + t_row) * Hq + kvh * G + (r % G)) * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + half * 4;
        const uint2 wv =
            make_uint2(pack_bf16x2(oacc[dt][g4 * 4 + 0] * inv, oacc[dt][g4 * 4 + 1] * inv),
                       pack_bf16x2(oacc[dt][g4 * 4 + 2] * inv, oacc[dt][g4 * 4 + 3] * inv));
        *reinterpret_cast<uint2*>(op + d) = wv;
      }
  }
}

}  // namespace pa
