// Device helpers shared by the gfx950 kernels: element types, 16-byte vector access, bf16
// conversion and wave64 cross-lane reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

constexpr int kWave = 64;
constexpr int kBlock = 16;                 // tokens per KV block supported by the kernels

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

// Storage tags: bf16 is carried as raw 16-bit patterns.
struct bf16_t { uint16_t bits; };

template <typename T> struct Elem;
template <> struct Elem<float> { static constexpr int kPerChunk = 4; };
template <> struct Elem<bf16_t> { static constexpr int kPerChunk = 8; };

__device__ __forceinline__ uint4 load16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}
__device__ __forceinline__ void store16(void* p, uint4 v) { *reinterpret_cast<uint4*>(p) = v; }

// Non-temporal 16-byte load for streamed-once data (KV slabs).
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
__device__ __forceinline__ uint4 load16_stream(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

__device__ __forceinline__ float u32_as_f32(uint32_t u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ uint32_t f32_as_u32(float f) { return __builtin_bit_cast(uint32_t, f); }

// Two bf16 packed in a dword -> two fp32 (exact).
__device__ __forceinline__ float bf16lo(uint32_t u) { return u32_as_f32(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return u32_as_f32(u & 0xffff0000u); }

// fp32 -> bf16, round to nearest even (hardware v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// dot of two packed bf16 pairs accumulated into fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                        __builtin_bit_cast(bf16x2_t, b), c, false);
}

// ---------------------------------------------------------------- DPP cross-lane movement
// dpp_ctrl encodings (GCN/CDNA DPP): quad_perm, row_half_mirror, row_ror.
constexpr int kDppQuadXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;  // lane i <-> 7-i inside each 8-lane half row
constexpr int kDppRowMirror = 0x140;      // lane i <-> 15-i inside each 16-lane row
constexpr int kDppRowRor8 = 0x128;        // rotate right by 8 inside each 16-lane row

template <int Ctrl>
__device__ __forceinline__ float dpp_f32(float v) {
  return u32_as_f32(__builtin_amdgcn_update_dpp(0, f32_as_u32(v), Ctrl, 0xF, 0xF, false));
}

// Sum over aligned groups of N lanes (N in 1,2,4,8,16,32,64); every lane gets its group's sum.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (N >= 2) v += dpp_f32<kDppQuadXor1>(v);
  if constexpr (N >= 4) v += dpp_f32<kDppQuadXor2>(v);
  if constexpr (N >= 8) v += dpp_f32<kDppRowHalfMirror>(v);
  if constexpr (N >= 16) v += dpp_f32<kDppRowMirror>(v);
  if constexpr (N >= 32) v += __shfl_xor(v, 16);
  if constexpr (N >= 64) v += __shfl_xor(v, 32);
  return v;
}

template <int N>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (N >= 2) v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  if constexpr (N >= 4) v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  if constexpr (N >= 8) v = fmaxf(v, dpp_f32<kDppRowHalfMirror>(v));
  if constexpr (N >= 16) v = fmaxf(v, dpp_f32<kDppRowMirror>(v));
  if constexpr (N >= 32) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (N >= 64) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

// Sum over lanes that share (lane % Stride) across the wave: xor over the bits >= Stride.
template <int Stride>
__device__ __forceinline__ float strided_sum(float v) {
  if constexpr (Stride <= 1) v += dpp_f32<kDppQuadXor1>(v);
  if constexpr (Stride <= 2) v += dpp_f32<kDppQuadXor2>(v);
  if constexpr (Stride <= 4) v += __shfl_xor(v, 4);
  if constexpr (Stride <= 8) v += dpp_f32<kDppRowRor8>(v);
  if constexpr (Stride <= 16) v += __shfl_xor(v, 16);
  if constexpr (Stride <= 32) v += __shfl_xor(v, 32);
  return v;
}

template <int Stride>
__device__ __forceinline__ float strided_max(float v) {
  if constexpr (Stride <= 1) v = fmaxf(v, dpp_f32<kDppQuadXor1>(v));
  if constexpr (Stride <= 2) v = fmaxf(v, dpp_f32<kDppQuadXor2>(v));
  if constexpr (Stride <= 4) v = fmaxf(v, __shfl_xor(v, 4));
  if constexpr (Stride <= 8) v = fmaxf(v, dpp_f32<kDppRowRor8>(v));
  if constexpr (Stride <= 16) v = fmaxf(v, __shfl_xor(v, 16));
  if constexpr (Stride <= 32) v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

}  // namespace pa
