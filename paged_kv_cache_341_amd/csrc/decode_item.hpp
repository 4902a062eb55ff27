// One decode split (sequence, kv head, split of consecutive blocks) as a device function, for
// the standalone decode kernel and the single-launch mixed kernel.  The algorithm is described
// at the top of pa_decode.hip.
#pragma once

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
  // blocks whose loads a wave keeps in flight together: 32 tokens' worth.  Measured against
  // 64 tokens' worth: fewer registers (93 instead of 125 at head_dim 128, 4 query heads per kv
  // head), five waves per SIMD instead of four, 2% faster on short batches and 7% on the beams.
  static constexpr int kBatch = B >= 32 ? 1 : 32 / B;
};

constexpr int kDecodeWaves = 4;
constexpr int kDecodeThreads = kDecodeWaves * kWave;

// Where the K (or V) rows of one (sequence, kv head) live.  The split item walks a sequence in
// units of U consecutive tokens (unit u holds positions u*U .. u*U+U-1); `unit` gives the base
// of unit u, uniform across the wave, and `row` the address of token k (0..U-1) of that unit.
//
// Every row policy has prepare(first, count, stride): the calling wave will visit units
// first, first + stride, ... (count of them, count <= 64), and may fetch what it needs for them
// up front.
//
// Paged, blocks of U tokens: unit u is physical block table[u] of the pool
// [blocks][num_kv_heads][U][D].  prepare() reads the wave's table entries once, one per lane
// (in the same round trip as the query rows), and unit() picks them with readlane, so no load
// batch waits on a table read.
template <typename T, int D, int U>
struct PagedRows {
  const int32_t* table;        // this sequence's block table
  int num_kv_heads, kvh;
  int first = 0, stride = 1;
  int ids = 0;                 // lane l: table[first + l * stride] (lanes < count)
  __device__ __forceinline__ void prepare(int first_unit, int count, int stride_units) {
    first = first_unit;
    stride = stride_units;
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    ids = lane < count ? table[first + lane * stride] : 0;
  }
  __device__ __forceinline__ const T* unit(const T* cache, int u) const {
    const int phys = __builtin_amdgcn_readlane(ids, wave_uniform((u - first) / stride));
    return cache + (static_cast<size_t>(phys) * num_kv_heads + kvh) * (static_cast<size_t>(U) * D);
  }
  __device__ __forceinline__ const T* row(const T*, const T* base, int, int k) const {
    return base + static_cast<size_t>(k) * D;
  }
};

// Paged, blocks of BT > U tokens (a block holds BT/U units): unit u is run u % (BT/U) of U rows
// of physical block table[u / (BT/U)].  The walk, its load batches and the split plan are then
// those of U-token blocks, so a split's four waves share its units evenly however large the
// blocks are.  prepare() reads one table entry per unit (neighbouring units repeat an entry).
template <typename T, int D, int U, int BT>
struct PagedLargeRows {
  static_assert(BT > U && BT % U == 0, "large blocks must hold whole units");
  static constexpr int kPer = BT / U;
  const int32_t* table;
  int num_kv_heads, kvh;
  int first = 0, stride = 1;
  // lane l: for unit v = first + l * stride (lanes < count), the index of its U-row run in the
  // pool counted for kv head 0: table[v / kPer] * num_kv_heads * kPer + v % kPer.  The run of
  // kv head h is that plus h * kPer.
  int runs = 0;
  __device__ __forceinline__ void prepare(int first_unit, int count, int stride_units) {
    first = first_unit;
    stride = stride_units;
    const int lane = static_cast<int>(threadIdx.x) % kWave;
    const unsigned v = static_cast<unsigned>(first + lane * stride);
    runs = lane < count ? table[v / kPer] * num_kv_heads * kPer + static_cast<int>(v % kPer) : 0;
  }
  __device__ __forceinline__ const T* unit(const T* cache, int u) const {
    const int run = __builtin_amdgcn_readlane(runs, wave_uniform((u - first) / stride));
    return cache + (static_cast<size_t>(run) + kvh * kPer) * (static_cast<size_t>(U) * D);
  }
  __device__ __forceinline__ const T* row(const T*, const T* base, int, int k) const {
    return base + static_cast<size_t>(k) * D;
  }
};

// Paged, blocks of BT < U tokens (a unit spans U/BT blocks): every lane looks up the block of
// the token it loads.  Tokens past the sequence end (the tail of its last unit) are read from
// its last token instead, so no table entry past ceil(len/BT) is touched; they are masked out
// by selection afterwards like every other tail slot.
template <typename T, int D, int U, int BT>
struct PagedSmallRows {
  static_assert(BT < U && U % BT == 0, "small blocks must tile a unit");
  const int32_t* table;
  int num_kv_heads, kvh, len;
  __device__ __forceinline__ void prepare(int, int, int) {}
  __device__ __forceinline__ const T* unit(const T* cache, int) const { return cache; }
  __device__ __forceinline__ const T* row(const T* cache, const T*, int u, int k) const {
    const int tok = min(u * U + k, len - 1);
    const int phys = table[tok / BT];
    return cache + ((static_cast<size_t>(phys) * num_kv_heads + kvh) * BT + tok % BT) * D;
  }
};

// Contiguous, no table: the cache is [num_seqs][num_kv_heads][capacity][D] with capacity a
// multiple of U, so every unit of a sequence lies inside its own slab.
template <typename T, int D, int U>
struct ContiguousRows {
  size_t slab;                 // element offset of (sequence, kv head, token 0)
  __device__ __forceinline__ void prepare(int, int, int) {}
  __device__ __forceinline__ const T* unit(const T* cache, int u) const {
    return cache + slab + static_cast<size_t>(u) * U * D;
  }
  __device__ __forceinline__ const T* row(const T*, const T* base, int, int k) const {
    return base + static_cast<size_t>(k) * D;
  }
};

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

// One split of one (sequence, kv head): `Waves` waves of the calling workgroup share it, and
// every one of them must make the call (it synchronises the workgroup).  B is the split walk's
// unit in tokens (the pool's block size for 8- and 16-token blocks; `Rows` maps a unit to its
// rows), and "block" in the body means such a unit.  `smem` holds
// max(plan.max_units() * B * G, Waves * G * D) floats (scores, then the waves' partial outputs), `red`
// Waves x G floats, `stat_m` and `stat_l` G floats each.
// `Batch` blocks per wave are loaded together before their math (0: 64 tokens' worth).
// With `Prio`, the K phase runs at wave priority 2 and the V phase at 0, each one band higher
// when `late` (a split dispatched late): splits that have made less progress issue first.
template <typename T, int D, int G, int B, int Waves, int Batch = 0, bool Prio = false,
          typename Rows>
__device__ __forceinline__ void decode_split_item(
    T* __restrict__ out, float* __restrict__ ws_ml, float* __restrict__ ws_acc,
    const T* __restrict__ q, const T* __restrict__ k_cache, const T* __restrict__ v_cache,
    Rows rows, int L, const int32_t* __restrict__ skip_blocks, int slot_base,
    int num_kv_heads, SplitPlan plan, int nsplit_max, float scale_log2, int s, int kvh,
    int split,
    float* smem, float (*red)[G], float* stat_m, float* stat_l, bool late = false) {
  using S = DecodeShape<T, D, G, B>;
  constexpr int kBlock = B;
  constexpr int kDecodeBatch = Batch > 0 ? Batch : S::kBatch;
  constexpr int kEpc = S::kEpc;
  constexpr int kThreadsW = Waves * kWave;
  const T tag{};
  float* logits = smem;                                  // [split tokens][G]

  const int nblk = (L + kBlock - 1) / kBlock;
  // leading blocks another kernel covers (a prefix shared with the sequence's group)
  const int skip = skip_blocks ? min(max(skip_blocks[s], 0), L / kBlock) : 0;
  const int b_begin = skip + plan.start(split);
  if (b_begin >= nblk) return;
  const int b_end = min(nblk, skip + plan.start(split + 1));
  const int ntok = min(L, b_end * kBlock) - b_begin * kBlock;
  const int nsplit_seq = plan.count(nblk - skip);
  const bool direct = skip == 0 && nsplit_seq == 1;   // the whole sequence in this split
  const int wave = wave_uniform(threadIdx.x / kWave);
  const int lane = threadIdx.x % kWave;
  const int Hq = num_kv_heads * G;

  if constexpr (Prio) {
    if (late) __builtin_amdgcn_s_setprio(3);
    else __builtin_amdgcn_s_setprio(2);
  }

  // this wave's units of the split: b_begin + wave, + Waves, ... below b_end
  rows.prepare(b_begin + wave, max(0, (b_end - b_begin - wave + Waves - 1) / Waves), Waves);

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
    for (int i0 = b_begin + wave; i0 < b_end; i0 += Waves * kDecodeBatch) {
      uint4 kr[kDecodeBatch][S::kTpb1][S::kR1];
#pragma unroll
      for (int j = 0; j < kDecodeBatch; ++j) {
        const int lb = i0 + j * Waves;
        if (lb < b_end) {
          const T* kb = rows.unit(k_cache, lb);
#pragma unroll
          for (int k = 0; k < S::kTpb1; ++k) {
            const T* kt = rows.row(k_cache, kb, lb, k * S::kGr1 + grp);
#pragma unroll
            for (int r = 0; r < S::kR1; ++r)
              kr[j][k][r] = load16_stream(kt + (sub + r * S::kW1) * kEpc);
          }
        }
      }
#pragma unroll
      for (int j = 0; j < kDecodeBatch; ++j) {
        const int lb = i0 + j * Waves;
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
    for (int t = threadIdx.x / G; t < ntok; t += kThreadsW / G)
      mx = fmaxf(mx, logits[t * G + h]);
    mx = strided_max<G>(mx);
    if (lane < G) red[wave][lane] = mx;
    __syncthreads();
    float m = red[0][h];
#pragma unroll
    for (int w = 1; w < Waves; ++w) m = fmaxf(m, red[w][h]);
    float sum = 0.f;
    for (int t = threadIdx.x / G; t < ntok; t += kThreadsW / G) {
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
      for (int w = 0; w < Waves; ++w) l += red[w][threadIdx.x];
      stat_m[threadIdx.x] = m;
      stat_l[threadIdx.x] = l;
    }
  }
  // the p values written above are read by other waves below
  __syncthreads();

  // ------------------------------------------------------------------ phase 3: p * V
  if constexpr (Prio) {
    if (late) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
  }
  const int grp = lane / S::kW3;
  const int sub = lane % S::kW3;
  float acc[G][S::kAcc];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < S::kAcc; ++e) acc[h][e] = 0.f;

  for (int i0 = b_begin + wave; i0 < b_end; i0 += Waves * kDecodeBatch) {
    uint4 vr[kDecodeBatch][S::kTpb3][S::kR3];
#pragma unroll
    for (int j = 0; j < kDecodeBatch; ++j) {
      const int lb = i0 + j * Waves;
      if (lb < b_end) {
        const T* vb = rows.unit(v_cache, lb);
#pragma unroll
        for (int k = 0; k < S::kTpb3; ++k) {
          const T* vt = rows.row(v_cache, vb, lb, k * S::kGr3 + grp);
#pragma unroll
          for (int r = 0; r < S::kR3; ++r)
            vr[j][k][r] = load16_stream(vt + (sub + r * S::kW3) * kEpc);
        }
      }
    }
#pragma unroll
    for (int j = 0; j < kDecodeBatch; ++j) {
      const int lb = i0 + j * Waves;
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
  for (int idx = threadIdx.x; idx < G * D; idx += kThreadsW) {
    const int h = idx / D;
    const int d = idx % D;
    float a = 0.f;
#pragma unroll
    for (int w = 0; w < Waves; ++w) a += wacc[(w * G + h) * D + d];
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

}  // namespace pa
