// Helpers of the MFMA attention kernels (prefill chunks and shared-prefix decode) for gfx950:
// swizzles of row-major K/V tiles in LDS, the transposing LDS read, buffer descriptors for
// buffer-to-LDS loads, and s_waitcnt immediates.
#pragma once

#include "device_common.hpp"

namespace pa {

constexpr uint32_t kRsrcWord3 = 0x00020000u;   // raw 32-bit buffer, gfx9 family

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8_t, v); }

// Row-major tiles of bf16 K or V rows of head_dim D in LDS, in 16-byte chunks, filled a 16-row
// block at a time by 1 KiB buffer-to-LDS loads (64 lanes x 16 bytes: kKeysPerLoad rows each).
// K rows are read one chunk per lane down 32 keys and V rows four keys at a time by the
// transposing load; the XOR swizzles spread both over the LDS banks.
template <int D>
struct KvTile {
  static_assert(D == 64 || D == 128 || D == 256, "head_dim");
  static constexpr int kChunks = D / 8;                        // 16-byte chunks per row
  static constexpr int kRowBytes = D * 2;
  static constexpr int kChunkBits = kChunks == 8 ? 3 : kChunks == 16 ? 4 : 5;
  static constexpr int kLoadsPerBlock = kBlock * kRowBytes / 1024;
  static constexpr int kKeysPerLoad = kWave / kChunks;
  static __device__ __forceinline__ int kswz(int key, int chunk) {
    return chunk ^ (key & (kChunks - 1));
  }
  static __device__ __forceinline__ int vswz(int key, int chunk) {
    return chunk ^ ((key & 3) << (kChunkBits - 2));
  }
};

typedef __attribute__((ext_vector_type(4))) short i16x4_t;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(3))) uint4 lds_uint4_t;

// Transposing LDS read of 8 bytes (gfx950 ds_read_b64_tr_b16): in each 16-lane group, lane i
// receives element i%4 of the 8-byte reads of lanes i/4, 4+i/4, 8+i/4 and 12+i/4.
__device__ __forceinline__ uint2 lds_read_tr16(const void* p) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_t*)(p));
  return __builtin_bit_cast(uint2, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A lane's value combined with the one lane l ^ 32 holds (the other half of the wave), through
// one v_permlane32_swap (gfx950): swapping x with itself leaves {x[l], x[l + 32]} in the lower
// half and {x[l - 32], x[l]} in the upper one, so the two results hold both values in every
// lane.  An LDS permute did this before (on the prefill's per-step row max, 1-2% of the kernel).
// max and + are commutative, so both halves get the same bits.
__device__ __forceinline__ float max_with_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Raw buffer descriptor over `bytes` bytes at `base`: loads past the end return zeros (and a
// buffer-to-LDS load writes zeros).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, kRsrcWord3);
}

// 16 bytes from a buffer straight into LDS, issued from inline assembly: lane l's data lands at
// LDS byte address lds_addr + 16 * l.  The compiler does not see this load, so it inserts no
// waits for it of its own (its tracking of buffer-to-LDS loads merges state across loop back
// edges and would drain the load pipeline before every tile); the caller orders the LDS
// accesses with explicit waits (wait_vmcnt_fence, lgkm_fence).  The memory clobber keeps the
// compiler from moving LDS accesses across it.  The vector-memory counter it raises only makes
// the compiler's own counted waits stricter, never looser.
// The load is non-temporal (nt): every tile it stages is read once per call.  Measured on the
// beam batch's shared prefix, the grouped call takes 80-81 us instead of 137-139 us when the
// caches were just filled with other, dirty data, and the same (73-74 us) when they were not.
__device__ __forceinline__ void buffer_to_lds16_untracked(__amdgpu_buffer_rsrc_t rsrc,
                                                          uint32_t lds_addr, int byte_offset) {
  asm volatile("s_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %0, %2, 0 offen nt lds"
               :
               : "v"(byte_offset), "s"(lds_addr), "s"(rsrc)
               : "memory", "m0");
}

// LDS byte address of an element of a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const uint4* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const lds_uint4_t*)p));
}

// s_waitcnt immediate that waits for vmcnt <= n only (gfx9 layout: vmcnt bits [3:0] and its
// high bits [15:14], expcnt [6:4] and lgkmcnt [11:8] left at their maxima).
constexpr int wait_vmcnt(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }
constexpr int kWaitVm0 = wait_vmcnt(0);
static_assert(wait_vmcnt(4) == 0x0F74 && wait_vmcnt(16) == 0x4F70, "s_waitcnt encoding");

// Explicit waits that are also compiler memory barriers (no memory access moves across them),
// for LDS tiles filled by buffer_to_lds16_untracked.
template <int N>
__device__ __forceinline__ void wait_vmcnt_fence() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}
__device__ __forceinline__ void lgkm_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

}  // namespace pa
