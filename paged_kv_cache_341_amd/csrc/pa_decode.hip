// Paged decode attention for gfx950.
//
// Operation: one query token per sequence attends to all of that sequence's cached tokens,
// which are gathered through its block table from 16-token blocks anywhere in the pool
// (cloudmash "Batching and PagedAttention", section "PagedAttention", step 4; study-docs
// "PagedAttention & Continuous Batching", section "Block tables").  Query head h reads kv head
// h / G, G = Hq / Hkv, so the G query heads of one kv head share every K/V byte read.
//
// Work split (our design, not from the pages): one workgroup of 4 waves per
// (sequence, kv head, split), a split being `bps` consecutive logical blocks.  Inside a split:
//   phase 1  each wave takes every 4th block, reads its K slab (16 x D contiguous elements),
//            computes the G scores of every token with lanes split over the head dimension
//            (DPP sums), and parks them in LDS;
//   phase 2  exact softmax statistics of the split: max and sum of exp2 per query head;
//   phase 3  each wave reads the V slabs of the same blocks and accumulates p * V in fp32,
//            lanes split over the head dimension again; waves are summed through LDS.
// A split with the whole sequence writes the normalised output; otherwise it writes
// (max, sum, unnormalised acc) and a merge kernel combines the splits in split order
// (log-sum-exp weighting), so results do not depend on scheduling.
// Only the last block of a sequence can be partly filled; its unfilled slots are masked by
// selection (score -inf, V treated as 0), never by multiplying, so garbage there is harmless.
#include "device_common.hpp"
#include "launch.hpp"

namespace pa {

template <typename T, int D, int G, int B>
struct DecodeShape {
  static constexpr int kEpc = Elem<T>::kPerChunk;   // elements per 16-byte chunk
  static constexpr int kCpr = D / kEpc;             // chunks per token row
  // phase 1 (scores): kW1 lanes share a token row, kR1 chunks each
  static constexpr int kW1 = 8;
  static constexpr int kR1 = kCpr / kW1;
  static constexpr int kGr1 = kWave / kW1;           // token groups per wave
  static constexpr int kTpb1 = B / kGr1;             // tokens per group per block
  // phase 3 (p * V): kW3 lanes share a token row, kR3 chunks each
  static constexpr int kW3 = kCpr >= 16 ? 16 : kCpr;
  static constexpr int kR3 = kCpr / kW3;
  static constexpr int kGr3 = kWave / kW3;
  static constexpr int kTpb3 = B / kGr3;
  static constexpr int kAcc = kR3 * kEpc;            // fp32 accumulators per head per lane
  static_assert(kCpr % kW1 == 0 && kCpr % kW3 == 0, "head_dim not supported");
  static_assert(kTpb1 >= 1 && kTpb3 >= 1, "bad lane split");
  // blocks whose loads a wave keeps in flight together: 64 tokens' worth
  static constexpr int kBatch = B >= 64 ? 1 : 64 / B;
};

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * kWave;

// Partial dot product of one 16-byte chunk of q with one chunk of K.
__device__ __forceinline__ float chunk_dot(uint4 q, uint4 k, float acc, bf16_t) {
  acc = dot2_bf16(q.x, k.x, acc);
  acc = dot2_bf16(q.y, k.y, acc);
  acc = dot2_bf16(q.z, k.z, acc);
  acc = dot2_bf16(q.w, k.w, acc);
  return acc;
}
__device__ __forceinline__ float chunk_dot(uint4 q, uint4 k, float acc, float) {
  acc = fmaf(u32_as_f32(q.x), u32_as_f32(k.x), acc);
  acc = fmaf(u32_as_f32(q.y), u32_as_f32(k.y), acc);
  acc = fmaf(u32_as_f32(q.z), u32_as_f32(k.z), acc);
  acc = fmaf(u32_as_f32(q.w), u32_as_f32(k.w), acc);
  return acc;
}

// Unpack a 16-byte chunk to fp32.
__device__ __forceinline__ void chunk_unpack(uint4 v, float* f, bf16_t) {
  f[0] = bf16lo(v.x); f[1] = bf16hi(v.x); f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
  f[4] = bf16lo(v.z); f[5] = bf16hi(v.z); f[6] = bf16lo(v.w); f[7] = bf16hi(v.w);
}
__device__ __forceinline__ void chunk_unpack(uint4 v, float* f, float) {
  f[0] = u32_as_f32(v.x); f[1] = u32_as_f32(v.y); f[2] = u32_as_f32(v.z); f[3] = u32_as_f32(v.w);
}

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(bf16_t* p, float v) {
  p->bits = static_cast<uint16_t>(pack_bf16x2(v, 0.f) & 0xffffu);
}

template <typename T, int D, int G, int B>
__global__ __launch_bounds__(kDecodeThreads) void pa_decode_split_kernel(
    T* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    const int32_t* __restrict__ skip_blocks, int slot_base, int num_kv_heads,
    int max_blocks_per_seq, int bps, int nsplit_max, float scale_log2) {
  using S = DecodeShape<T, D, G, B>;
  constexpr int kBlock = B;
  constexpr int kDecodeBatch = S::kBatch;
  constexpr int kEpc = S::kEpc;
  constexpr int kCpr = S::kCpr;
  const T tag{};
  extern __shared__ float smem[];
  float* logits = smem;                                  // [bps*16][G]
  __shared__ float red[kDecodeWaves][G];
  __shared__ float stat_m[G];
  __shared__ float stat_l[G];

  // grid.x runs over (sequence, kv head) and grid.y over splits, so consecutive workgroups
  // belong to different kv heads.  Workgroups are dealt to the 8 XCDs round-robin in launch
  // order; with this order each XCD gets an even share of every split index (instead of one
  // XCD holding every sequence's first split), and the beams that share a block read it
  // through the same XCD's L2.
  const int kvh = blockIdx.x % num_kv_heads;
  const int s = blockIdx.x / num_kv_heads;
  const int split = blockIdx.y;
  const int L = seq_lens[s];
  const int nblk = (L + kBlock - 1) / kBlock;
  // leading blocks another kernel covers (a prefix shared with the sequence's group)
  const int skip = skip_blocks ? min(max(skip_blocks[s], 0), L / kBlock) : 0;
  const int b_begin = skip + split * bps;
  if (b_begin >= nblk) return;
  const int b_end = min(nblk, b_begin + bps);
  const int ntok = min(L, b_end * kBlock) - b_begin * kBlock;
  const int nsplit_seq = (nblk - skip + bps - 1) / bps;
  const bool direct = skip == 0 && nsplit_seq == 1;   // the whole sequence in this split
  const int wave = wave_uniform(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int Hq = num_kv_heads * G;
  const int32_t* table = block_tables + static_cast<size_t>(s) * max_blocks_per_seq;
  const size_t slab = static_cast<size_t>(kBlock) * D;   // elements per (block, kv head)

  // ---------------------------------------------------------------- phase 1: scores
  {
    const int grp = lane / S::kW1;
    const int sub = lane % S::kW1;
    uint4 qr[G][S::kR1];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const T* qh = q + (static_cast<size_t>(s) * Hq + kvh * G + h) * D;
#pragma unroll
      for (int r = 0; r < S::kR1; ++r) qr[h][r] = load16(qh + (sub + r * S::kW1) * kEpc);
    }
    for (int i0 = b_begin + wave; i0 < b_end; i0 += kDecodeWaves * kDecodeBatch) {
      uint4 kr[kDecodeBatch][S::kTpb1][S::kR1];
#pragma unroll
      for (int j = 0; j < kDecodeBatch; ++j) {
        const int lb = i0 + j * kDecodeWaves;
        if (lb < b_end) {
          const int phys = wave_uniform(table[lb]);
          const T* kb = k_cache + (static_cast<size_t>(phys) * num_kv_heads + kvh) * slab;
#pragma unroll
          for (int k = 0; k < S::kTpb1; ++k)
#pragma unroll
            for (int r = 0; r < S::kR1; ++r)
              kr[j][k][r] = load16_stream(
                  kb + ((k * S::kGr1 + grp) * kCpr + sub + r * S::kW1) * kEpc);
        }
      }
#pragma unroll
      for (int j = 0; j < kDecodeBatch; ++j) {
        const int lb = i0 + j * kDecodeWaves;
        if (lb < b_end) {
#pragma unroll
          for (int k = 0; k < S::kTpb1; ++k) {
            const int tok = lb * kBlock + k * S::kGr1 + grp;     // absolute position
            const int rel = tok - b_begin * kBlock;
#pragma unroll
            for (int h = 0; h < G; ++h) {
              float acc = 0.f;
#pragma unroll
              for (int r = 0; r < S::kR1; ++r) acc = chunk_dot(qr[h][r], kr[j][k][r], acc, tag);
              float sc = group_sum<S::kW1>(acc) * scale_log2;
              sc = tok < L ? sc : kNegInf;
              if (sub == (k * G + h) % S::kW1) logits[rel * G + h] = sc;
            }
          }
        }
      }
    }
  }
  __syncthreads();

  // ---------------------------------------------------- phase 2: split softmax statistics
  {
    const int h = threadIdx.x % G;
    float mx = kNegInf;
    for (int t = threadIdx.x / G; t < ntok; t += kDecodeThreads / G)
      mx = fmaxf(mx, logits[t * G + h]);
    mx = strided_max<G>(mx);
    if (lane < G) red[wave][lane] = mx;
    __syncthreads();
    float m = red[0][h];
#pragma unroll
    for (int w = 1; w < kDecodeWaves; ++w) m = fmaxf(m, red[w][h]);
    float sum = 0.f;
    for (int t = threadIdx.x / G; t < ntok; t += kDecodeThreads / G) {
      const float p = exp2f(logits[t * G + h] - m);
      logits[t * G + h] = p;
      sum += p;
    }
    sum = strided_sum<G>(sum);
    __syncthreads();                         // everyone has read red[] for the max
    if (lane < G) red[wave][lane] = sum;
    __syncthreads();
    if (threadIdx.x < G) {
      float l = 0.f;
#pragma unroll
      for (int w = 0; w < kDecodeWaves; ++w) l += red[w][threadIdx.x];
      stat_m[threadIdx.x] = m;
      stat_l[threadIdx.x] = l;
    }
  }
  // the p values written above are read by other waves below
  __syncthreads();

  // ------------------------------------------------------------------ phase 3: p * V
  const int grp = lane / S::kW3;
  const int sub = lane % S::kW3;
  float acc[G][S::kAcc];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < S::kAcc; ++e) acc[h][e] = 0.f;

  for (int i0 = b_begin + wave; i0 < b_end; i0 += kDecodeWaves * kDecodeBatch) {
    uint4 vr[kDecodeBatch][S::kTpb3][S::kR3];
#pragma unroll
    for (int j = 0; j < kDecodeBatch; ++j) {
      const int lb = i0 + j * kDecodeWaves;
      if (lb < b_end) {
        const int phys = wave_uniform(table[lb]);
        const T* vb = v_cache + (static_cast<size_t>(phys) * num_kv_heads + kvh) * slab;
#pragma unroll
        for (int k = 0; k < S::kTpb3; ++k)
#pragma unroll
          for (int r = 0; r < S::kR3; ++r)
            vr[j][k][r] =
                load16_stream(vb + ((k * S::kGr3 + grp) * kCpr + sub + r * S::kW3) * kEpc);
      }
    }
#pragma unroll
    for (int j = 0; j < kDecodeBatch; ++j) {
      const int lb = i0 + j * kDecodeWaves;
      if (lb < b_end) {
        const bool partial = (lb + 1) * kBlock > L;
#pragma unroll
        for (int k = 0; k < S::kTpb3; ++k) {
          const int tok = lb * kBlock + k * S::kGr3 + grp;
          const int rel = tok - b_begin * kBlock;
          float p[G];
#pragma unroll
          for (int h = 0; h < G; ++h) p[h] = logits[rel * G + h];
          if (partial && tok >= L) {
#pragma unroll
            for (int h = 0; h < G; ++h) p[h] = 0.f;
#pragma unroll
            for (int r = 0; r < S::kR3; ++r) vr[j][k][r] = make_uint4(0, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < S::kR3; ++r) {
            float v[kEpc];
            chunk_unpack(vr[j][k][r], v, tag);
#pragma unroll
            for (int e = 0; e < kEpc; ++e)
#pragma unroll
              for (int h = 0; h < G; ++h) acc[h][r * kEpc + e] = fmaf(p[h], v[e], acc[h][r * kEpc + e]);
          }
        }
      }
    }
  }
  // sum the token groups of this wave (lanes sharing `sub`)
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < S::kAcc; ++e) acc[h][e] = strided_sum<S::kW3>(acc[h][e]);

  __syncthreads();                           // logits no longer needed: reuse LDS
  float* wacc = smem;                        // [waves][G][D]
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int r = 0; r < S::kR3; ++r)
#pragma unroll
        for (int e = 0; e < kEpc; ++e)
          wacc[(wave * G + h) * D + (sub + r * S::kW3) * kEpc + e] = acc[h][r * kEpc + e];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < G * D; idx += kDecodeThreads) {
    const int h = idx / D;
    const int d = idx % D;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < kDecodeWaves; ++w) a += wacc[(w * G + h) * D + d];
    const size_t row = static_cast<size_t>(s) * Hq + kvh * G + h;
    if (direct) {
      store_out(out + row * D + d, a / stat_l[h]);
    } else {
      const size_t slot = row * nsplit_max + slot_base + split;
      ws_acc[slot * D + d] = a;
      if (d == 0) {
        ws_ml[slot * 2 + 0] = stat_m[h];
        ws_ml[slot * 2 + 1] = stat_l[h];
      }
    }
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
    int slot_base, int shared_split_keys, int num_rows, int num_q_heads, int bps,
    int nsplit_max) {
  constexpr int kPer = D / kWave;
  const int row = blockIdx.x * kMergeWaves + static_cast<int>(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  if (row >= num_rows) return;
  const int s = row / num_q_heads;
  const int L = seq_lens[s];
  const int nblk = (L + B - 1) / B;
  // partials of this row: the shared-prefix splits end at slot_base, the splits of the rest
  // start there, so they form one range
  const int skip = skip_blocks ? min(max(skip_blocks[s], 0), L / B) : 0;
  const int ns = skip > 0 ? (skip * B + shared_split_keys - 1) / shared_split_keys : 0;
  const int nt = (nblk - skip + bps - 1) / bps;
  if (ns == 0 && nt <= 1) return;                 // written directly by the split kernel
  const int nsplit = ns + nt;
  const float* ml = ws_ml + (static_cast<size_t>(row) * nsplit_max + slot_base - ns) * 2;
  const float* acc = ws_acc + (static_cast<size_t>(row) * nsplit_max + slot_base - ns) * D;

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

template <typename T, int D, int G, int B>
hipError_t launch_decode_tb(const DecodeArgs& a) {
  const size_t lds = std::max<size_t>(static_cast<size_t>(a.bps) * B * G,
                                      static_cast<size_t>(kDecodeWaves) * G * D) * sizeof(float);
  const dim3 grid_split(a.num_seqs * a.num_kv_heads, a.nsplit_tail);
  hipLaunchKernelGGL((pa_decode_split_kernel<T, D, G, B>), grid_split, dim3(kDecodeThreads),
                     lds, a.stream, static_cast<T*>(a.out), a.ws_ml, a.ws_acc,
                     static_cast<const T*>(a.q), static_cast<const T*>(a.k_cache),
                     static_cast<const T*>(a.v_cache), a.block_tables, a.seq_lens,
                     a.skip_blocks, a.slot_base, a.num_kv_heads, a.max_blocks_per_seq, a.bps,
                     a.nsplit_max, a.scale_log2);
  if (a.nsplit_max > 1) {
    const int rows = a.num_seqs * a.num_kv_heads * G;
    hipLaunchKernelGGL((pa_decode_merge_kernel<T, D, B>),
                       dim3((rows + kMergeWaves - 1) / kMergeWaves), dim3(kMergeWaves * kWave), 0,
                       a.stream, static_cast<T*>(a.out), a.ws_ml, a.ws_acc, a.seq_lens,
                       a.skip_blocks, a.slot_base, a.shared_split_keys, rows,
                       a.num_kv_heads * G, a.bps, a.nsplit_max);
  }
  return hipGetLastError();
}

template <typename T, int D, int G>
hipError_t launch_decode_t(const DecodeArgs& a) {
  switch (a.block_size) {
    case 8: return launch_decode_tb<T, D, G, 8>(a);
    case 16: return launch_decode_tb<T, D, G, 16>(a);
    case 32: return launch_decode_tb<T, D, G, 32>(a);
    case 64: return launch_decode_tb<T, D, G, 64>(a);
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
