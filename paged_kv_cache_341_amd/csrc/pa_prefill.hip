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
//   * Rows of a tile are (token, query head) pairs with the G heads of one kv head innermost, so
//     the G heads share every K/V tile.  A workgroup owns 128 rows: 4 waves x 32 rows.
//   * Keys go through LDS 64 at a time (four 16-token blocks, looked up in the table once per
//     tile).  K is stored row-major with a 16-byte XOR swizzle; V is stored transposed
//     ([head_dim][key]) with an 8-byte XOR swizzle, because the MFMA operand for P.V needs
//     consecutive keys of one head-dim column in a lane.
//   * Scores are computed transposed, S^T = K Q^T, so a lane holds one query row: the running
//     max / sum and the rescale of the output accumulator are per-lane scalars, and the
//     probabilities are already laid out as the B operand of O^T = V^T P^T.  P is rounded to
//     bf16 for that product; everything else stays fp32.
//   * Masking is by selection (-inf scores, zero-filled K/V past the sequence end), applied
//     only to tiles that reach past a row's position.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

namespace {

constexpr int kD = 128;
constexpr int kRowsPerWave = 32;
constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;
constexpr int kTileRows = kWaves * kRowsPerWave;   // 128
constexpr int kKvTile = 64;                         // keys per LDS tile (4 blocks)
constexpr int kChunks = kD / 8;                     // 16-byte chunks per K row

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// 8-byte-group swizzle of the transposed V tile: row d, key group kg (4 keys).
__device__ __forceinline__ int vt_group(int d, int kg) { return kg ^ (((d >> 1) ^ (d >> 3)) & 15); }

}  // namespace

template <int G>
__global__ __launch_bounds__(kThreads, 2) void pa_prefill_kernel(
    bf16_t* __restrict__ out, const bf16_t* __restrict__ q, const bf16_t* __restrict__ k_cache,
    const bf16_t* __restrict__ v_cache, const int32_t* __restrict__ block_tables,
    const int32_t* __restrict__ seq_lens, const int32_t* __restrict__ query_start_loc,
    int num_kv_heads, int max_blocks_per_seq, float scale_log2) {
  constexpr int kTokPerTile = kTileRows / G;
  __shared__ uint4 sK[kKvTile * kChunks];            // 16 KiB
  __shared__ uint32_t sVT[kD * kKvTile / 2];         // 16 KiB

  const int tile = blockIdx.x;
  const int kvh = blockIdx.y;
  const int c = blockIdx.z;
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

  const int tid = threadIdx.x;
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

  f32x16_t oacc[kD / 32];
#pragma unroll
  for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) oacc[dt][v] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;

  for (int kt = 0; kt < num_kv_tiles; ++kt) {
    // ------------------------------------------------------------- stage K and V^T in LDS
    __syncthreads();
    {
      int phys[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const int lb = kt * 4 + b;
        phys[b] = lb < nblk ? wave_uniform(table[lb]) : 0;
      }
      // K: thread -> (block j, slot tid/16, chunk tid%16); one wave reads 4 whole rows
      const int slot = tid >> 4;
      const int ch = tid & 15;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = j * kBlock + slot;
        uint4 val = make_uint4(0, 0, 0, 0);
        if (kt * kKvTile + key < L) {
          const bf16_t* kp = k_cache +
              (static_cast<size_t>(phys[j]) * num_kv_heads + kvh) * slab + slot * kD + ch * 8;
          val = load16(kp);
        }
        sK[key * kChunks + (ch ^ (key & 15))] = val;
      }
      // V: thread -> (key pair, chunk); two keys' chunks are interleaved into key-pair words
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int kp2 = (tid >> 4) + 16 * j;      // key pair 0..31
        const int k0 = 2 * kp2;
        const int b = k0 >> 4;
        const int sl = k0 & 15;
        int pb = phys[0];
        pb = b == 1 ? phys[1] : pb;
        pb = b == 2 ? phys[2] : pb;
        pb = b == 3 ? phys[3] : pb;
        const bf16_t* vp =
            v_cache + (static_cast<size_t>(pb) * num_kv_heads + kvh) * slab + sl * kD + ch * 8;
        const int kabs = kt * kKvTile + k0;
        uint4 v0 = make_uint4(0, 0, 0, 0), v1 = make_uint4(0, 0, 0, 0);
        if (kabs < L) v0 = load16(vp);
        if (kabs + 1 < L) v1 = load16(vp + kD);
        const uint32_t a[4] = {v0.x, v0.y, v0.z, v0.w};
        const uint32_t bb[4] = {v1.x, v1.y, v1.z, v1.w};
        const int kg = k0 >> 2;
        const int wsub = (k0 >> 1) & 1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = ch * 8 + e;
          const uint32_t lo = a[e / 2], hi = bb[e / 2];
          const uint32_t w = (e & 1) ? ((lo >> 16) | (hi & 0xffff0000u))
                                     : ((lo & 0xffffu) | (hi << 16));
          sVT[d * (kKvTile / 2) + vt_group(d, kg) * 2 + wsub] = w;
        }
      }
    }
    __syncthreads();
    if (kt * kKvTile >= kv_end_w) continue;     // all keys of this tile are in this wave's future

    // ----------------------------------------------------------------- S^T = K Q^T
    f32x16_t sacc[2];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2) {
#pragma unroll
      for (int v = 0; v < 16; ++v) sacc[t2][v] = 0.f;
      const int key = t2 * 32 + col;
#pragma unroll
      for (int ks = 0; ks < kD / 16; ++ks) {
        const int chn = ks * 2 + half;
        const uint4 a = sK[key * kChunks + (chn ^ (key & 15))];
        sacc[t2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(qreg[ks]),
                                                           sacc[t2], 0, 0, 0);
      }
    }

    // ----------------------------------------------------------------- online softmax
    const bool need_mask = kt * kKvTile + kKvTile - 1 > prefix + t_lo_w;
    float x[32];
#pragma unroll
    for (int t2 = 0; t2 < 2; ++t2)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        float s = sacc[t2][v] * scale_log2;
        if (need_mask) {
          const int key = kt * kKvTile + t2 * 32 + (v / 4) * 8 + half * 4 + (v % 4);
          s = key <= pos ? s : kNegInf;
        }
        x[t2 * 16 + v] = s;
      }
    float mx = x[0];
#pragma unroll
    for (int i = 1; i < 32; ++i) mx = fmaxf(mx, x[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    m_run = m_new;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      x[i] = exp2f(x[i] - m_new);
      psum += x[i];
    }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int v = 0; v < 16; ++v) oacc[dt][v] *= alpha;

    // P^T operand for k-step s: the lane's own scores v = (s%2)*8 .. +8 of key subtile s/2
    uint4 pT[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const float* p = x + (s / 2) * 16 + (s % 2) * 8;
      pT[s] = make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                         pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7]));
    }

    // ----------------------------------------------------------------- O^T += V^T P^T
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt) {
      const int d = dt * 32 + col;
      const uint32_t* row = sVT + d * (kKvTile / 2);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int kg0 = 8 * (s / 2) + 4 * (s % 2) + half;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + vt_group(d, kg0) * 2);
        const uint2 hi = *reinterpret_cast<const uint2*>(row + vt_group(d, kg0 + 2) * 2);
        const uint4 a = make_uint4(lo.x, lo.y, hi.x, hi.y);
        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(as_bf16x8(a), as_bf16x8(pT[s]),
                                                           oacc[dt], 0, 0, 0);
      }
    }
  }

  // ------------------------------------------------------------------------- write out
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = 1.f / l_tot;
  if (row_valid) {
    bf16_t* op = out + (static_cast<size_t>(q0 + t_row) * Hq + kvh * G + (r % G)) * kD;
#pragma unroll
    for (int dt = 0; dt < kD / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + g4 * 8 + half * 4;
        const uint2 w = make_uint2(pack_bf16x2(oacc[dt][g4 * 4 + 0] * inv, oacc[dt][g4 * 4 + 1] * inv),
                                   pack_bf16x2(oacc[dt][g4 * 4 + 2] * inv, oacc[dt][g4 * 4 + 3] * inv));
        *reinterpret_cast<uint2*>(op + d) = w;
      }
  }
}

template <int G>
static hipError_t launch_prefill_g(const PrefillArgs& a) {
  const int tiles = (a.max_q_len * G + kTileRows - 1) / kTileRows;
  const dim3 grid(tiles, a.num_kv_heads, a.num_chunks);
  hipLaunchKernelGGL((pa_prefill_kernel<G>), grid, dim3(kThreads), 0, a.stream,
                     static_cast<bf16_t*>(a.out), static_cast<const bf16_t*>(a.q),
                     static_cast<const bf16_t*>(a.k_cache), static_cast<const bf16_t*>(a.v_cache),
                     a.block_tables, a.seq_lens, a.query_start_loc, a.num_kv_heads,
                     a.max_blocks_per_seq, a.scale_log2);
  return hipGetLastError();
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
