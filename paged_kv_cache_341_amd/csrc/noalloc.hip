// pa_decode_noalloc: pa_decode with its split partials in a library-owned static device array
// instead of a caller workspace, for callers that cannot allocate device memory (code under
// graph capture, serving loops that forbid allocation).  Declared in include/pagedattn.h.
//
// The array lives in this file's device code object, so every GPU the library runs on holds
// its own copy, from the first call on that GPU until the process ends.  Its device address is
// looked up once per device, with that device current, and only that address is ever passed
// to a kernel: in host code the array's name is a host-side stand-in, not a device pointer.
// Calls on one GPU share the array, so calls that overlap on that GPU (on different streams,
// or from different threads) race on it; the decode kernels need it uninitialised.
#include <hip/hip_runtime.h>

#include <mutex>

#include "errors.hpp"
#include "pagedattn.h"

namespace {

constexpr size_t kScratchBytes = PA_DECODE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};

DeviceScratch g_scratch[kMaxDevices];

// Device address of `scratch` on the current device (looked up on the first call there).
hipError_t scratch_on_current_device(void** ptr, int* device) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  DeviceScratch& d = g_scratch[dev];
  std::call_once(d.once, [&d] {
    void* p = nullptr;
    d.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    d.ptr = d.err == hipSuccess ? p : nullptr;
  });
  *ptr = d.ptr;
  *device = dev;
  return d.err;
}

}  // namespace

extern "C" {

pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                            pa_dtype dtype, void* stream) {
  // Size check first: it needs no device, and a refused call enqueues nothing.
  const size_t need = pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                               block_size, max_seq_len);
  if (need > kScratchBytes)
    return pa::fail(PA_ERR_WORKSPACE_TOO_SMALL,
                    "pa_decode_noalloc: these sizes need %zu bytes of split partials; the "
                    "library's static scratch holds %zu (use pa_decode with a workspace)",
                    need, kScratchBytes);
  void* ws = nullptr;
  int dev = -1;
  const hipError_t e = scratch_on_current_device(&ws, &dev);
  if (e != hipSuccess)
    return pa::fail(PA_ERR_DEVICE, "pa_decode_noalloc: address of the static scratch on "
                    "device %d: %s", dev, hipGetErrorString(e));
  // Every other check, the split plan and the launches are pa_decode's own.
  return pa_decode(out, q, k_cache, v_cache, block_tables, seq_lens, num_seqs, num_q_heads,
                   num_kv_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                   max_seq_len, scale, dtype, ws, kScratchBytes, stream);
}

}  // extern "C"
