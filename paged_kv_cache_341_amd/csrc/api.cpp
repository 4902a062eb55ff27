// C ABI of the paged KV-cache library: argument checks, split planning, dispatch.
// Every check here runs on host scalars and pointers only, before any HIP call, so a rejected
// call enqueues nothing.  The entry points are declared and documented in include/pagedattn.h.
#include "pagedattn.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>

#include "checked.hpp"
#include "errors.hpp"
#include "launch.hpp"

namespace pa {

namespace {
thread_local std::string g_last_error;
}  // namespace

pa_status fail(pa_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

pa_status ok() {
  g_last_error.clear();
  return PA_OK;
}

const char* last_error() { return g_last_error.c_str(); }

}  // namespace pa

namespace {

using pa::fail;
using pa::ok;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int elem_bytes(pa_dtype d) { return d == PA_DTYPE_BF16 ? 2 : 4; }

bool valid_dtype(pa_dtype d) { return d == PA_DTYPE_F32 || d == PA_DTYPE_BF16; }

bool supported_group(int g) { return g == 1 || g == 2 || g == 4 || g == 8; }

constexpr int kSupportedBlock = 16;

// Block sizes the decode kernels are built for (tokens per block).
bool decode_block_supported(int b) {
  return b == 1 || b == 4 || b == 8 || b == 16 || b == 32 || b == 64;
}

// Tokens per unit of the decode split walk: the block size for 8- and 16-token blocks, else 16:
// blocks smaller than 8 tokens are looked up token by token, blocks larger than 16 are walked
// 16 tokens at a time, and contiguous KV (block_size 0 here) as 16-token blocks.
int decode_unit(int block_size) { return block_size == 8 || block_size == 16 ? block_size : 16; }

// Tokens per unit of the contiguous decode (the same walk as 16-token paged blocks).
constexpr int kContiguousUnit = 16;

constexpr int kMaxSplitBlocks = 256;

// Blocks per decode split.  A split covers 256, 512 or 1024 tokens, the smallest that keeps
// the number of workgroups near kTargetGroups when every sequence is max_seq_len long; the LDS
// score buffer caps a split at 8192/G tokens.  PA_DECODE_SPLIT_BLOCKS overrides the block
// count (tuning aid).
int plan_blocks_per_split(int num_seqs, int num_kv_heads, int group, int block_size,
                          int max_seq_len) {
  const int nblk = (max_seq_len + block_size - 1) / block_size;
  static const int env = [] {
    const char* e = std::getenv("PA_DECODE_SPLIT_BLOCKS");
    return e ? std::atoi(e) : 0;
  }();
  const int cap = std::max(1, 8192 / group / block_size);
  int bps;
  if (env > 0) {
    bps = env;
  } else {
    constexpr long kTargetGroups = 4096;
    const long want_tokens = (static_cast<long>(max_seq_len) * num_seqs * num_kv_heads +
                              kTargetGroups - 1) / kTargetGroups;
    int tokens = 256;
    while (tokens < want_tokens && tokens < 1024) tokens *= 2;
    bps = std::max(1, tokens / block_size);
  }
  bps = std::min(bps, cap);
  // a wave of a split keeps its table entries one per lane: at most 64 per wave, and the split
  // kernels run at least 4 waves per split
  bps = std::min(bps, kMaxSplitBlocks);
  bps = std::max(bps, 1);
  return std::min(bps, std::max(nblk, 1));
}

// The split plan of pa_decode and pa_decode_contiguous.  With b = plan_blocks_per_split's
// size and n = ceil(max units / b) splits of a longest sequence:
//  * 3 <= n <= 16 and at least 2048 workgroups in a uniform grid: shrinking sizes, first
//    max(1, n / 8) splits of 2b, then two of b, then b / 2 to the end.  Workgroups of split
//    index j start after all of index j - 1 (the dispatch order), so the pieces dispatched last
//    are the smallest and the kernel's tail is short: measured on ragged batches of 64-256
//    sequences (lengths U[128, 4096] and lognormal up to 16384) and on 128 beams of about
//    4200 tokens, 3-4% faster than one size.  It is not used for longer sequences (32 splits
//    of equal-length sequences already balance) or grids that fit the chip about once (the
//    bigger first pieces lengthen the critical path).
//  * otherwise every split has b units.
// PA_DECODE_SPLIT_PLAN="s0,c0,s1,c1,s2" overrides it (tuning aid; sizes non-increasing, the
// largest within the caps above).
pa::SplitPlan plan_decode_splits(int num_seqs, int num_kv_heads, int group, int unit,
                                 int max_seq_len) {
  const int bps = plan_blocks_per_split(num_seqs, num_kv_heads, group, unit, max_seq_len);
  static const pa::SplitPlan env = [] {
    pa::SplitPlan p{0, 0, 0, 0, 0};
    const char* e = std::getenv("PA_DECODE_SPLIT_PLAN");
    if (e && std::sscanf(e, "%d,%d,%d,%d,%d", &p.s0, &p.c0, &p.s1, &p.c1, &p.s2) != 5)
      p = pa::SplitPlan{0, 0, 0, 0, 0};
    return p;
  }();
  const int cap = std::min(kMaxSplitBlocks, std::max(1, 8192 / group / unit));
  if (env.s2 > 0 && env.s0 >= env.s1 && env.s1 >= env.s2 && env.c0 >= 0 && env.c1 >= 0 &&
      env.s0 <= cap)
    return env;
  const int nblk = (max_seq_len + unit - 1) / unit;
  const int n = (nblk + bps - 1) / bps;
  const int64_t grid = static_cast<int64_t>(num_seqs) * num_kv_heads * n;
  if (n >= 3 && n <= 16 && grid >= 2048 && bps >= 2)
    return pa::SplitPlan{std::min(2 * bps, cap), std::max(1, n / 8), bps, 2, bps / 2};
  return pa::SplitPlan::uniform(bps);
}

size_t decode_ws_bytes(int num_seqs, int num_q_heads, int head_dim, int nsplit) {
  if (nsplit <= 1) return 0;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * nsplit;
  const size_t ml = (rows * 2 * sizeof(float) + 255) & ~size_t(255);
  return ml + rows * head_dim * sizeof(float);
}

pa_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(PA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

// In checked mode, run a host-side check of device contents; a violation fails the call with
// PA_ERR_INVALID_ARGUMENT before anything is enqueued.
#define PA_CHECK_CONTENTS(name, expr)                                                      \
  do {                                                                                     \
    if (pa::checked::enabled()) {                                                          \
      const std::string msg_ = (expr);                                                     \
      if (!msg_.empty())                                                                   \
        return fail(PA_ERR_INVALID_ARGUMENT, "%s (checked mode): %s", name, msg_.c_str()); \
    }                                                                                      \
  } while (0)

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
  switch (s) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARGUMENT: return "PA_ERR_INVALID_ARGUMENT";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED";
    case PA_ERR_WORKSPACE_TOO_SMALL: return "PA_ERR_WORKSPACE_TOO_SMALL";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE";
  }
  return "PA_ERR_UNKNOWN";
}

const char* pa_last_error(void) { return pa::last_error(); }

int pa_set_checked_mode(int enable) { return pa::checked::set_enabled(enable != 0) ? 1 : 0; }

int pa_checked_mode(void) { return pa::checked::enabled() ? 1 : 0; }

size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_seq_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      !decode_block_supported(block_size) || max_seq_len <= 0 ||
      num_q_heads % num_kv_heads != 0)
    return 0;
  const int g = num_q_heads / num_kv_heads;
  const int unit = decode_unit(block_size);
  const pa::SplitPlan plan = plan_decode_splits(num_seqs, num_kv_heads, g, unit, max_seq_len);
  const int nsplit = plan.count((max_seq_len + unit - 1) / unit);
  return decode_ws_bytes(num_seqs, num_q_heads, head_dim, nsplit);
}

pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens, int32_t num_seqs,
                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                    int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                    int32_t max_seq_len, float scale, pa_dtype dtype, void* workspace,
                    size_t workspace_bytes, void* stream) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: null pointer argument");
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: sizes must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: num_q_heads %d not a multiple of "
                "num_kv_heads %d", num_q_heads, num_kv_heads);
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: unknown dtype");
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: max_seq_len %d exceeds table capacity %lld",
                max_seq_len, static_cast<long long>(max_blocks_per_seq) * block_size);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: q, out and caches must be 16-byte aligned");
  if (!(scale > 0.f) || scale == __builtin_inff())
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: scale must be finite and positive");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: head_dim %d (supported: 64, 128, 256)", head_dim);
  if (!decode_block_supported(block_size))
    return fail(PA_ERR_UNSUPPORTED,
                "pa_decode: block_size %d (supported: 1, 4, 8, 16, 32, 64)", block_size);
  const int g = num_q_heads / num_kv_heads;
  if (!supported_group(g))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: %d query heads per kv head (supported: 1,2,4,8)",
                g);
  const int unit = decode_unit(block_size);
  const pa::SplitPlan plan = plan_decode_splits(num_seqs, num_kv_heads, g, unit, max_seq_len);
  const int nsplit = plan.count((max_seq_len + unit - 1) / unit);
  const size_t need = decode_ws_bytes(num_seqs, num_q_heads, head_dim, nsplit);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "pa_decode: workspace %zu bytes, need %zu",
                workspace_bytes, need);
  if (need > 0 && !aligned16(workspace))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode: workspace must be 16-byte aligned");
  // grid: x = num_seqs * num_kv_heads workgroups of 256 lanes, y = splits
  if (nsplit > 65535 || static_cast<int64_t>(num_seqs) * num_kv_heads > (int64_t{1} << 24))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode: grid too large");

  PA_CHECK_CONTENTS("pa_decode",
                    pa::checked::tables(static_cast<hipStream_t>(stream), block_tables, seq_lens,
                                        num_seqs, max_blocks_per_seq, num_blocks, block_size,
                                        max_seq_len));

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * nsplit;
  a.ws_ml = need ? static_cast<float*>(workspace) : nullptr;
  a.ws_acc = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             ((rows * 2 * sizeof(float) + 255) & ~size_t(255)))
                  : nullptr;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.plan = plan;
  a.nsplit_max = nsplit;
  a.nsplit_tail = nsplit;
  a.skip_blocks = nullptr;
  a.slot_base = 0;
  a.shared_split_keys = 1;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.bf16 = dtype == PA_DTYPE_BF16;
  a.stream = static_cast<hipStream_t>(stream);
  return device_status(pa::launch_decode(a), "pa_decode launch");
}

pa_status pa_decode_contiguous(void* out, const void* q, const void* k, const void* v,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t capacity,
                               int32_t max_seq_len, float scale, pa_dtype dtype,
                               void* workspace, size_t workspace_bytes, void* stream) {
  if (!out || !q || !k || !v || !seq_lens)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_contiguous: null pointer argument");
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      capacity <= 0 || max_seq_len <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_contiguous: sizes must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_contiguous: num_q_heads %d not a multiple "
                "of num_kv_heads %d", num_q_heads, num_kv_heads);
  if (!valid_dtype(dtype))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_contiguous: unknown dtype");
  if (capacity % kContiguousUnit != 0 || max_seq_len > capacity)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_contiguous: capacity %d must be a multiple "
                "of %d and at least max_seq_len %d", capacity, kContiguousUnit, max_seq_len);
  if (!aligned16(out) || !aligned16(q) || !aligned16(k) || !aligned16(v))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_contiguous: buffers must be 16-byte aligned");
  if (!(scale > 0.f) || scale == __builtin_inff())
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_contiguous: scale must be finite and "
                "positive");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_contiguous: head_dim %d (supported: 64, 128, "
                "256)", head_dim);
  const int g = num_q_heads / num_kv_heads;
  if (!supported_group(g))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_contiguous: %d query heads per kv head "
                "(supported: 1,2,4,8)", g);
  const pa::SplitPlan plan =
      plan_decode_splits(num_seqs, num_kv_heads, g, kContiguousUnit, max_seq_len);
  const int nsplit = plan.count((max_seq_len + kContiguousUnit - 1) / kContiguousUnit);
  const size_t need = decode_ws_bytes(num_seqs, num_q_heads, head_dim, nsplit);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "pa_decode_contiguous: workspace %zu bytes, need "
                "%zu", workspace_bytes, need);
  if (need > 0 && !aligned16(workspace))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_contiguous: workspace must be 16-byte "
                "aligned");
  if (nsplit > 65535 || static_cast<int64_t>(num_seqs) * num_kv_heads > (int64_t{1} << 24))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_contiguous: grid too large");
  PA_CHECK_CONTENTS("pa_decode_contiguous",
                    pa::checked::tables(static_cast<hipStream_t>(stream), nullptr, seq_lens,
                                        num_seqs, 0, 0, kContiguousUnit, max_seq_len));

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k;
  a.v_cache = v;
  a.block_tables = nullptr;
  a.seq_lens = seq_lens;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * nsplit;
  a.ws_ml = need ? static_cast<float*>(workspace) : nullptr;
  a.ws_acc = need ? reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                             ((rows * 2 * sizeof(float) + 255) & ~size_t(255)))
                  : nullptr;
  a.contiguous = true;
  a.capacity = capacity;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = kContiguousUnit;
  a.max_blocks_per_seq = 0;
  a.plan = plan;
  a.nsplit_max = nsplit;
  a.nsplit_tail = nsplit;
  a.skip_blocks = nullptr;
  a.slot_base = 0;
  a.shared_split_keys = 1;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.bf16 = dtype == PA_DTYPE_BF16;
  a.stream = static_cast<hipStream_t>(stream);
  return device_status(pa::launch_decode(a), "pa_decode_contiguous launch");
}

// ------------------------------------------------------------------------- grouped decode
namespace {

// Largest number of shared keys one shared-prefix work item takes: the kernel keeps a split's
// block ids one per lane (at most 64 blocks).
constexpr int kSharedSplitMax = 64 * 16;
constexpr int kSharedSplitMin = 64;
constexpr int64_t kComputeUnits = 256;

// Shared keys per split.  Fewer, longer splits mean fewer partials to write and merge (on 16
// prompts x 8 beams over 4096 shared tokens, 1024-key splits take 68 us per grouped call warm
// against 73 us at 512 keys), so splits are as long as possible while the shared-prefix launch
// still has at least one work item per compute unit.  Its work items are (row tile of 32 rows,
// kv head, split); num_seqs x G / 32 row tiles per kv head is the fewest the groups can have,
// and max_seq_len bounds the shared length, so the estimate is a lower bound on the items.
int plan_shared_split_keys(int num_seqs, int g, int num_kv_heads, int max_seq_len) {
  const int64_t tiles = (static_cast<int64_t>(num_seqs) * g + 31) / 32 * num_kv_heads;
  int keys = kSharedSplitMax;
  while (keys > kSharedSplitMin && tiles * ((max_seq_len + keys - 1) / keys) < kComputeUnits)
    keys /= 2;
  return keys;
}

struct GroupedPlan {
  int bps, shared_split_keys, nsplit_shared, nsplit_tail, nsplit_max;
  size_t ml_bytes, total;
};

GroupedPlan plan_grouped(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                         int block_size, int max_seq_len) {
  GroupedPlan p{};
  const int g = num_q_heads / num_kv_heads;
  p.bps = plan_blocks_per_split(num_seqs, num_kv_heads, g, block_size, max_seq_len);
  const int nblk = (max_seq_len + block_size - 1) / block_size;
  p.nsplit_tail = (nblk + p.bps - 1) / p.bps;
  p.shared_split_keys = plan_shared_split_keys(num_seqs, g, num_kv_heads, max_seq_len);
  p.nsplit_shared = (max_seq_len + p.shared_split_keys - 1) / p.shared_split_keys;
  p.nsplit_max = p.nsplit_shared + p.nsplit_tail;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * p.nsplit_max;
  p.ml_bytes = (rows * 2 * sizeof(float) + 255) & ~size_t(255);
  p.total = p.ml_bytes + rows * head_dim * sizeof(float);
  return p;
}

}  // namespace

size_t pa_decode_grouped_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_seq_len) {
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 ||
      block_size != kSupportedBlock || max_seq_len <= 0 || num_q_heads % num_kv_heads != 0)
    return 0;
  return plan_grouped(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len)
      .total;
}

pa_status pa_decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            const int32_t* group_start, const int32_t* shared_blocks,
                            int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_seq_len, float scale, pa_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !group_start ||
      !shared_blocks)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: null pointer argument");
  if (num_seqs <= 0 || num_groups <= 0 || max_group_size <= 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0 ||
      max_blocks_per_seq <= 0 || max_seq_len <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: sizes must be positive");
  if (num_groups > num_seqs || max_group_size > num_seqs)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: more groups or members than "
                "sequences");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: num_q_heads %d not a multiple of "
                "num_kv_heads %d", num_q_heads, num_kv_heads);
  if (!valid_dtype(dtype))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: unknown dtype");
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: max_seq_len exceeds table capacity");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: buffers must be 16-byte aligned");
  if (!(scale > 0.f) || scale == __builtin_inff())
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: scale must be finite and positive");
  if (dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_grouped: only bf16 is supported");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_grouped: head_dim %d (supported: 64, 128, 256)",
                head_dim);
  if (block_size != kSupportedBlock)
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_grouped: block_size %d (supported: 16)",
                block_size);
  const int g = num_q_heads / num_kv_heads;
  if (!supported_group(g))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_grouped: %d query heads per kv head "
                "(supported: 1,2,4,8)", g);
  const GroupedPlan p =
      plan_grouped(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, max_seq_len);
  if (!workspace || workspace_bytes < p.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "pa_decode_grouped: workspace %zu bytes, need %zu",
                workspace_bytes, p.total);
  if (!aligned16(workspace))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_decode_grouped: workspace must be 16-byte aligned");
  const int row_tiles = (max_group_size * g + 31) / 32;
  if (p.nsplit_max > 65535 || static_cast<int64_t>(num_seqs) * num_kv_heads > (int64_t{1} << 24) ||
      static_cast<int64_t>(num_groups) * row_tiles * num_kv_heads > (int64_t{1} << 26))
    return fail(PA_ERR_UNSUPPORTED, "pa_decode_grouped: grid too large");

  float* ws_ml = static_cast<float*>(workspace);
  float* ws_acc = reinterpret_cast<float*>(static_cast<char*>(workspace) + p.ml_bytes);
  const float scale_log2 = scale * 1.4426950408889634f;
  hipStream_t st = static_cast<hipStream_t>(stream);
  PA_CHECK_CONTENTS("pa_decode_grouped",
                    pa::checked::tables(st, block_tables, seq_lens, num_seqs, max_blocks_per_seq,
                                        num_blocks, block_size, max_seq_len));
  PA_CHECK_CONTENTS("pa_decode_grouped",
                    pa::checked::groups(st, group_start, shared_blocks, block_tables, seq_lens,
                                        num_seqs, num_groups, max_group_size, max_blocks_per_seq,
                                        block_size));

  pa::SharedPrefixArgs sp{};
  sp.ws_ml = ws_ml;
  sp.ws_acc = ws_acc;
  sp.q = q;
  sp.k_cache = k_cache;
  sp.v_cache = v_cache;
  sp.block_tables = block_tables;
  sp.group_start = group_start;
  sp.shared_blocks = shared_blocks;
  sp.seq_lens = seq_lens;
  sp.num_seqs = num_seqs;
  sp.num_groups = num_groups;
  sp.num_q_heads = num_q_heads;
  sp.num_kv_heads = num_kv_heads;
  sp.head_dim = head_dim;
  sp.max_blocks_per_seq = max_blocks_per_seq;
  sp.row_tiles = row_tiles;
  sp.nsplit_shared = p.nsplit_shared;
  sp.split_keys = p.shared_split_keys;
  sp.slot_base = p.nsplit_shared;
  sp.nsplit_max = p.nsplit_max;
  sp.scale_log2 = scale_log2;
  sp.stream = st;
  hipError_t e = pa::launch_shared_prefix(sp);
  if (e != hipSuccess) return device_status(e, "pa_decode_grouped shared-prefix launch");

  pa::DecodeArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.ws_ml = ws_ml;
  a.ws_acc = ws_acc;
  a.num_seqs = num_seqs;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.plan = pa::SplitPlan::uniform(p.bps);
  a.nsplit_max = p.nsplit_max;
  a.nsplit_tail = p.nsplit_tail;
  a.skip_blocks = shared_blocks;
  a.slot_base = p.nsplit_shared;
  a.shared_split_keys = p.shared_split_keys;
  a.scale_log2 = scale_log2;
  a.bf16 = true;
  a.stream = st;
  return device_status(pa::launch_decode(a), "pa_decode_grouped launch");
}

size_t pa_prefill_workspace_size(int32_t, int32_t, int32_t, int32_t, int32_t) { return 0; }

// ------------------------------------------------------------------------- mixed step
namespace {

constexpr size_t kMixedHeader = 256;     // work counters
constexpr int kMixedMaxChunks = 128;
constexpr int kMixedMaxSeqs = 2048;
constexpr int kMixedMaxSplits = 2047;    // split slots per decode sequence

struct MixedPlan {
  pa::SplitPlan plan;
  int nsplit;
  size_t ml_bytes, total;
};

MixedPlan plan_mixed(int num_seqs, int num_q_heads, int num_kv_heads, int head_dim,
                     int block_size, int dec_max_seq_len) {
  MixedPlan p{};
  if (num_seqs <= 0) {
    p.plan = pa::SplitPlan::uniform(1);
    p.nsplit = 1;
    p.total = kMixedHeader;
    return p;
  }
  // the standalone decode's plan, so the decode splits shrink toward the last-dispatched ones
  const int g = num_q_heads / num_kv_heads;
  p.plan = plan_decode_splits(num_seqs, num_kv_heads, g, block_size, dec_max_seq_len);
  p.nsplit = p.plan.count((dec_max_seq_len + block_size - 1) / block_size);
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * p.nsplit;
  p.ml_bytes = (rows * 2 * sizeof(float) + 255) & ~size_t(255);
  p.total = kMixedHeader + (p.nsplit > 1 ? p.ml_bytes + rows * head_dim * sizeof(float) : 0);
  return p;
}

}  // namespace

size_t pa_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t dec_max_seq_len) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 ||
      (head_dim != 64 && head_dim != 128 && head_dim != 256) || block_size != kSupportedBlock || num_q_heads % num_kv_heads != 0 ||
      (num_seqs > 0 && dec_max_seq_len <= 0))
    return 0;
  return plan_mixed(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, dec_max_seq_len)
      .total;
}

pa_status pa_mixed_step(const pa_mixed_batch* b, void* workspace, size_t workspace_bytes,
                        void* stream) {
  if (!b) return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: null batch");
  if (b->num_new_tokens < 0 || b->num_chunks < 0 || b->num_seqs < 0 || b->num_q_heads <= 0 ||
      b->num_kv_heads <= 0 || b->head_dim <= 0 || b->block_size <= 0 || b->num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: sizes must be positive (counts >= 0)");
  if (b->num_q_heads % b->num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: num_q_heads %d not a multiple of "
                "num_kv_heads %d", b->num_q_heads, b->num_kv_heads);
  if (!valid_dtype(b->dtype)) return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: unknown dtype");
  if (!b->k_cache || !b->v_cache || !aligned16(b->k_cache) || !aligned16(b->v_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: pools must be non-null and 16-byte "
                "aligned");
  if (!(b->scale > 0.f) || b->scale == __builtin_inff())
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: scale must be finite and positive");
  if (b->num_new_tokens > 0 &&
      (!b->k_new || !b->v_new || !b->slot_mapping || !aligned16(b->k_new) || !aligned16(b->v_new)))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: append buffers null or misaligned");
  if (b->num_chunks > 0) {
    if (!b->chunk_out || !b->chunk_q || !b->chunk_tables || !b->chunk_seq_lens ||
        !b->query_start_loc || !aligned16(b->chunk_out) || !aligned16(b->chunk_q))
      return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: chunk buffers null or misaligned");
    if (b->chunk_total_q <= 0 || b->chunk_max_q_len <= 0 || b->chunk_max_seq_len <= 0 ||
        b->chunk_max_blocks_per_seq <= 0 || b->chunk_max_q_len > b->chunk_total_q ||
        b->chunk_max_q_len > b->chunk_max_seq_len ||
        static_cast<int64_t>(b->chunk_max_seq_len) >
            static_cast<int64_t>(b->chunk_max_blocks_per_seq) * b->block_size)
      return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: inconsistent chunk bounds");
  }
  if (b->num_seqs > 0) {
    if (!b->dec_out || !b->dec_q || !b->dec_tables || !b->dec_seq_lens ||
        !aligned16(b->dec_out) || !aligned16(b->dec_q))
      return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: decode buffers null or misaligned");
    if (b->dec_max_seq_len <= 0 || b->dec_max_blocks_per_seq <= 0 ||
        static_cast<int64_t>(b->dec_max_seq_len) >
            static_cast<int64_t>(b->dec_max_blocks_per_seq) * b->block_size)
      return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: inconsistent decode bounds");
  }
  if (b->dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_mixed_step: only bf16 is supported");
  if ((b->head_dim != 64 && b->head_dim != 128 && b->head_dim != 256) ||
      b->block_size != kSupportedBlock)
    return fail(PA_ERR_UNSUPPORTED, "pa_mixed_step: head_dim %d, block_size %d (supported: "
                "64, 128 or 256; 16)", b->head_dim, b->block_size);
  const int g = b->num_q_heads / b->num_kv_heads;
  if (!supported_group(g))
    return fail(PA_ERR_UNSUPPORTED, "pa_mixed_step: %d query heads per kv head (supported: "
                "1,2,4,8)", g);
  if (b->num_chunks > kMixedMaxChunks || b->num_seqs > kMixedMaxSeqs)
    return fail(PA_ERR_UNSUPPORTED, "pa_mixed_step: %d chunks, %d decode sequences (at most %d "
                "and %d)", b->num_chunks, b->num_seqs, kMixedMaxChunks, kMixedMaxSeqs);
  const MixedPlan p = plan_mixed(b->num_seqs, b->num_q_heads, b->num_kv_heads, b->head_dim,
                                 b->block_size, b->dec_max_seq_len);
  if (p.nsplit > kMixedMaxSplits)
    return fail(PA_ERR_UNSUPPORTED, "pa_mixed_step: %d decode splits per sequence (at most %d)",
                p.nsplit, kMixedMaxSplits);
  if (!workspace || workspace_bytes < p.total)
    return fail(PA_ERR_WORKSPACE_TOO_SMALL, "pa_mixed_step: workspace %zu bytes, need %zu",
                workspace_bytes, p.total);
  if (!aligned16(workspace))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_mixed_step: workspace must be 16-byte aligned");
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      cus <= 0)
    return fail(PA_ERR_DEVICE, "pa_mixed_step: cannot read the device's compute-unit count");

  hipStream_t st = static_cast<hipStream_t>(stream);
  if (b->num_new_tokens > 0)
    PA_CHECK_CONTENTS("pa_mixed_step", pa::checked::slots(st, b->slot_mapping, b->num_new_tokens,
                                                          b->num_blocks, b->block_size));
  if (b->num_chunks > 0) {
    PA_CHECK_CONTENTS("pa_mixed_step chunks",
                      pa::checked::chunks(st, b->query_start_loc, b->chunk_seq_lens,
                                          b->num_chunks, b->chunk_total_q, b->chunk_max_q_len));
    PA_CHECK_CONTENTS("pa_mixed_step chunks",
                      pa::checked::tables(st, b->chunk_tables, b->chunk_seq_lens, b->num_chunks,
                                          b->chunk_max_blocks_per_seq, b->num_blocks,
                                          b->block_size, b->chunk_max_seq_len));
  }
  if (b->num_seqs > 0)
    PA_CHECK_CONTENTS("pa_mixed_step decodes",
                      pa::checked::tables(st, b->dec_tables, b->dec_seq_lens, b->num_seqs,
                                          b->dec_max_blocks_per_seq, b->num_blocks,
                                          b->block_size, b->dec_max_seq_len));
  int* queues = static_cast<int*>(workspace);
  char* ws = static_cast<char*>(workspace) + kMixedHeader;
  float* ws_ml = reinterpret_cast<float*>(ws);
  float* ws_acc = reinterpret_cast<float*>(ws + p.ml_bytes);

  // 1. append, which also zeroes the two work counters
  pa::AppendArgs ap{};
  ap.k_cache = b->k_cache;
  ap.v_cache = b->v_cache;
  ap.k_new = b->k_new;
  ap.v_new = b->v_new;
  ap.slot_mapping = b->slot_mapping;
  ap.num_tokens = b->num_new_tokens;
  ap.num_kv_heads = b->num_kv_heads;
  ap.head_dim = b->head_dim;
  ap.block_size = b->block_size;
  ap.elem_bytes = 2;
  ap.zero_words = queues;
  ap.num_zero_words = 2;
  ap.stream = st;
  hipError_t e = pa::launch_append(ap);
  if (e != hipSuccess) return device_status(e, "pa_mixed_step append launch");
  if (b->num_chunks == 0 && b->num_seqs == 0) return ok();

  // 2. chunks and decode splits in one launch
  pa::MixedArgs m{};
  m.chunk_out = b->chunk_out;
  m.chunk_q = b->chunk_q;
  m.chunk_tables = b->chunk_tables;
  m.chunk_seq_lens = b->chunk_seq_lens;
  m.query_start_loc = b->query_start_loc;
  m.num_chunks = b->num_chunks;
  m.chunk_max_blocks_per_seq = b->chunk_max_blocks_per_seq;
  m.dec_out = b->dec_out;
  m.dec_q = b->dec_q;
  m.dec_tables = b->dec_tables;
  m.dec_seq_lens = b->dec_seq_lens;
  m.num_seqs = b->num_seqs;
  m.dec_max_blocks_per_seq = b->dec_max_blocks_per_seq;
  m.plan = p.plan;
  m.nsplit_max = p.nsplit;
  m.ws_ml = ws_ml;
  m.ws_acc = ws_acc;
  m.queues = queues;
  m.k_cache = b->k_cache;
  m.v_cache = b->v_cache;
  m.num_q_heads = b->num_q_heads;
  m.num_kv_heads = b->num_kv_heads;
  m.head_dim = b->head_dim;
  m.num_workgroups = cus;
  m.scale_log2 = b->scale * 1.4426950408889634f;
  m.stream = st;
  e = pa::launch_mixed(m);
  if (e != hipSuccess) return device_status(e, "pa_mixed_step mixed launch");
  if (b->num_seqs == 0 || p.nsplit <= 1) return ok();

  // 3. merge of the decode splits
  pa::DecodeArgs d{};
  d.out = b->dec_out;
  d.ws_ml = ws_ml;
  d.ws_acc = ws_acc;
  d.seq_lens = b->dec_seq_lens;
  d.num_seqs = b->num_seqs;
  d.num_q_heads = b->num_q_heads;
  d.num_kv_heads = b->num_kv_heads;
  d.head_dim = b->head_dim;
  d.block_size = b->block_size;
  d.plan = p.plan;
  d.nsplit_max = p.nsplit;
  d.nsplit_tail = p.nsplit;
  d.skip_blocks = nullptr;
  d.slot_base = 0;
  d.shared_split_keys = 1;
  d.stream = st;
  return device_status(pa::launch_decode_merge(d), "pa_mixed_step merge launch");
}

pa_status pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* query_start_loc, int32_t num_chunks, int32_t total_q,
                           int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                           pa_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream) {
  (void)workspace;
  (void)workspace_bytes;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens || !query_start_loc)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_prefill_chunk: null pointer argument");
  if (num_chunks <= 0 || total_q <= 0 || max_q_len <= 0 || max_seq_len <= 0 ||
      num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_blocks <= 0 || max_blocks_per_seq <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_prefill_chunk: sizes must be positive");
  if (num_q_heads % num_kv_heads != 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_prefill_chunk: num_q_heads %d not a multiple of "
                "num_kv_heads %d", num_q_heads, num_kv_heads);
  if (max_q_len > total_q || max_q_len > max_seq_len)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_prefill_chunk: max_q_len exceeds total_q or "
                "max_seq_len");
  if (!valid_dtype(dtype))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_prefill_chunk: unknown dtype");
  if (static_cast<int64_t>(max_seq_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_prefill_chunk: max_seq_len exceeds table capacity");
  if (!aligned16(out) || !aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_prefill_chunk: buffers must be 16-byte aligned");
  if (!(scale > 0.f) || scale == __builtin_inff())
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_prefill_chunk: scale must be finite and positive");
  if (dtype != PA_DTYPE_BF16)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: only bf16 is supported");
  if (head_dim != 64 && head_dim != 128 && head_dim != 256)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: head_dim %d (supported: 64, 128, 256)",
                head_dim);
  if (block_size != kSupportedBlock)
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: block_size %d (supported: 16)",
                block_size);
  const int g = num_q_heads / num_kv_heads;
  if (!supported_group(g))
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: %d query heads per kv head "
                "(supported: 1,2,4,8)", g);
  // one workgroup per (chunk, row tile, kv head): row tiles of 256 rows (128 at head_dim 256);
  // rows are (token, query head) pairs
  const int64_t tile_rows = head_dim == 256 ? 128 : 256;
  const int64_t tiles_max =
      (static_cast<int64_t>(max_q_len) * (num_q_heads / num_kv_heads) + tile_rows - 1) /
      tile_rows;
  if (static_cast<int64_t>(num_chunks) * tiles_max * num_kv_heads > (int64_t{1} << 24))
    return fail(PA_ERR_UNSUPPORTED, "pa_prefill_chunk: grid too large");
  PA_CHECK_CONTENTS("pa_prefill_chunk",
                    pa::checked::chunks(static_cast<hipStream_t>(stream), query_start_loc,
                                        seq_lens, num_chunks, total_q, max_q_len));
  PA_CHECK_CONTENTS("pa_prefill_chunk",
                    pa::checked::tables(static_cast<hipStream_t>(stream), block_tables, seq_lens,
                                        num_chunks, max_blocks_per_seq, num_blocks, block_size,
                                        max_seq_len));
  pa::PrefillArgs a{};
  a.out = out;
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.query_start_loc = query_start_loc;
  a.num_chunks = num_chunks;
  a.total_q = total_q;
  a.max_q_len = max_q_len;
  a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.max_blocks_per_seq = max_blocks_per_seq;
  a.scale_log2 = scale * 1.4426950408889634f;
  a.stream = static_cast<hipStream_t>(stream);
  return device_status(pa::launch_prefill(a), "pa_prefill_chunk launch");
}

pa_status kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                    void* stream) {
  if (num_tokens < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "kv_append: sizes must be positive (num_tokens >= 0)");
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARGUMENT, "kv_append: unknown dtype");
  if (num_tokens == 0) return ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return fail(PA_ERR_INVALID_ARGUMENT, "kv_append: null pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return fail(PA_ERR_INVALID_ARGUMENT, "kv_append: buffers must be 16-byte aligned");
  if ((head_dim * elem_bytes(dtype)) % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "kv_append: head_dim rows must be a multiple of 16 bytes");
  PA_CHECK_CONTENTS("kv_append", pa::checked::slots(static_cast<hipStream_t>(stream),
                                                    slot_mapping, num_tokens, num_blocks,
                                                    block_size));
  pa::AppendArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.k_new = k_new;
  a.v_new = v_new;
  a.slot_mapping = slot_mapping;
  a.num_tokens = num_tokens;
  a.num_kv_heads = num_kv_heads;
  a.head_dim = head_dim;
  a.block_size = block_size;
  a.elem_bytes = elem_bytes(dtype);
  a.stream = static_cast<hipStream_t>(stream);
  return device_status(pa::launch_append(a), "kv_append launch");
}

pa_status cow_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                          int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 || num_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT,
                "cow_copy_blocks: sizes must be positive (num_pairs >= 0)");
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARGUMENT, "cow_copy_blocks: unknown dtype");
  if (num_pairs == 0) return ok();
  if (!k_cache || !v_cache || !block_pairs)
    return fail(PA_ERR_INVALID_ARGUMENT, "cow_copy_blocks: null pointer argument");
  if (!aligned16(k_cache) || !aligned16(v_cache))
    return fail(PA_ERR_INVALID_ARGUMENT, "cow_copy_blocks: caches must be 16-byte aligned");
  const int64_t block_bytes =
      static_cast<int64_t>(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "cow_copy_blocks: block bytes must be a multiple of 16");
  PA_CHECK_CONTENTS("cow_copy_blocks",
                    pa::checked::pairs(static_cast<hipStream_t>(stream), block_pairs, num_pairs,
                                       num_blocks, num_blocks, true));
  pa::CowArgs a{};
  a.dst_k = k_cache;
  a.dst_v = v_cache;
  a.src_k = k_cache;
  a.src_v = v_cache;
  a.pairs = block_pairs;
  a.num_pairs = num_pairs;
  a.block_bytes = block_bytes;
  a.stream = static_cast<hipStream_t>(stream);
  return device_status(pa::launch_cow(a), "cow_copy_blocks launch");
}

pa_status swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                      const int64_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_src_blocks,
                      int32_t num_dst_blocks, pa_dtype dtype, void* stream) {
  if (num_pairs < 0 || num_kv_heads <= 0 || head_dim <= 0 || block_size <= 0 ||
      num_src_blocks <= 0 || num_dst_blocks <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "swap_blocks: sizes must be positive (num_pairs >= 0)");
  if (!valid_dtype(dtype)) return fail(PA_ERR_INVALID_ARGUMENT, "swap_blocks: unknown dtype");
  if (num_pairs == 0) return ok();
  if (!dst_k || !dst_v || !src_k || !src_v || !block_pairs)
    return fail(PA_ERR_INVALID_ARGUMENT, "swap_blocks: null pointer argument");
  if (!aligned16(dst_k) || !aligned16(dst_v) || !aligned16(src_k) || !aligned16(src_v))
    return fail(PA_ERR_INVALID_ARGUMENT, "swap_blocks: pools must be 16-byte aligned");
  if (dst_k == src_k || dst_v == src_v)
    return fail(PA_ERR_INVALID_ARGUMENT, "swap_blocks: source and destination pools are the "
                "same (use cow_copy_blocks)");
  const int64_t block_bytes =
      static_cast<int64_t>(num_kv_heads) * block_size * head_dim * elem_bytes(dtype);
  if (block_bytes % 16 != 0)
    return fail(PA_ERR_UNSUPPORTED, "swap_blocks: block bytes must be a multiple of 16");
  PA_CHECK_CONTENTS("swap_blocks",
                    pa::checked::pairs(static_cast<hipStream_t>(stream), block_pairs, num_pairs,
                                       num_src_blocks, num_dst_blocks, false));
  pa::CowArgs a{};
  a.dst_k = dst_k;
  a.dst_v = dst_v;
  a.src_k = src_k;
  a.src_v = src_v;
  a.pairs = block_pairs;
  a.num_pairs = num_pairs;
  a.block_bytes = block_bytes;
  a.stream = static_cast<hipStream_t>(stream);
  return device_status(pa::launch_cow(a), "swap_blocks launch");
}

pa_status pa_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink,
                            int32_t num_workgroups, void* stream) {
  if (!src || !sink) return fail(PA_ERR_INVALID_ARGUMENT, "pa_hbm_read_probe: null pointer");
  if (bytes == 0 || bytes % 16 != 0 || !aligned16(src))
    return fail(PA_ERR_INVALID_ARGUMENT,
                "pa_hbm_read_probe: bytes must be a positive multiple of 16, src 16-byte aligned");
  if (num_workgroups <= 0 || num_workgroups > (1 << 20))
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_hbm_read_probe: num_workgroups out of range");
  return device_status(pa::launch_hbm_probe(src, bytes, sink, num_workgroups,
                                            static_cast<hipStream_t>(stream)),
                       "pa_hbm_read_probe launch");
}

pa_status pa_mfma_probe(float* sink, int32_t num_workgroups, int32_t iters, void* stream) {
  if (!sink) return fail(PA_ERR_INVALID_ARGUMENT, "pa_mfma_probe: null pointer");
  if (num_workgroups <= 0 || num_workgroups > (1 << 20) || iters <= 0)
    return fail(PA_ERR_INVALID_ARGUMENT, "pa_mfma_probe: num_workgroups or iters out of range");
  return device_status(pa::launch_mfma_probe(sink, num_workgroups, iters,
                                             static_cast<hipStream_t>(stream)),
                       "pa_mfma_probe launch");
}

}  // extern "C"
