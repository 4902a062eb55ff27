// Native host-side block manager: free stacks, block tables, reference counts, fork,
// copy-on-write decisions, admission in blocks, and preemption by swap or recompute.  The
// operations and the readings where the pages are silent are documented in
// include/block_manager.h; every call either completes or changes nothing.
#include "block_manager.h"

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <map>
#include <new>
#include <string>
#include <unordered_map>
#include <unordered_set>
#include <vector>

namespace {

thread_local std::string g_bm_error;

pa_bm_status bm_fail(pa_bm_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
pa_bm_status bm_fail(pa_bm_status st, const char* fmt, ...) {
  char buf[256];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_bm_error = buf;
  return st;
}

pa_bm_status bm_ok() {
  g_bm_error.clear();
  return PA_BM_OK;
}

struct Seq {
  std::vector<int32_t> blocks;
  int64_t length = 0;
  int64_t request = -1;
  int32_t state = PA_BM_RUNNING;
  int64_t recompute_tokens = 0;
};

// One pool: a free stack (top = back) and reference counts.
struct Pool {
  std::vector<int32_t> free_stack;
  std::vector<int32_t> ref;

  bool init(int32_t n, const int32_t* order) {
    ref.assign(static_cast<size_t>(n), 0);
    free_stack.resize(static_cast<size_t>(n));
    std::vector<char> seen(static_cast<size_t>(n), 0);
    for (int32_t i = 0; i < n; ++i) {
      const int32_t b = order ? order[i] : i;
      if (b < 0 || b >= n || seen[static_cast<size_t>(b)]) return false;
      seen[static_cast<size_t>(b)] = 1;
      free_stack[static_cast<size_t>(n - 1 - i)] = b;   // order[0] ends on top
    }
    return true;
  }
  int32_t num_free() const { return static_cast<int32_t>(free_stack.size()); }
  int32_t pop() {
    const int32_t b = free_stack.back();
    free_stack.pop_back();
    return b;
  }
};

}  // namespace

struct pa_bm {
  int32_t block_size = 16;
  Pool gpu, cpu;
  std::unordered_map<int64_t, Seq> seqs;
  std::map<int64_t, std::vector<int64_t>> requests;   // request id (= arrival) -> members
  int64_t next_request = 0;
  pa_bm_stats st{};

  int32_t pop_gpu() {
    const int32_t b = gpu.pop();
    gpu.ref[static_cast<size_t>(b)] = 1;
    ++st.blocks_allocated;
    return b;
  }
  void release_gpu(int32_t b) {
    if (--gpu.ref[static_cast<size_t>(b)] == 0) {
      gpu.free_stack.push_back(b);
      ++st.blocks_freed;
    }
  }
  int64_t blocks_for(int64_t tokens) const { return (tokens + block_size - 1) / block_size; }

  int64_t blocks_needed(const Seq& s, int64_t num_new) const {
    int64_t need = blocks_for(s.length + num_new) - static_cast<int64_t>(s.blocks.size());
    if (num_new > 0 && s.length % block_size != 0 &&
        gpu.ref[static_cast<size_t>(s.blocks.back())] > 1)
      need += 1;
    return need;
  }

  // Grow a resident sequence; the caller has checked the free count.
  void append(Seq& s, int64_t num_new, int64_t* slots, int64_t* pairs, int32_t* npairs) {
    int32_t np = 0;
    for (int64_t t = 0; t < num_new; ++t) {
      const int64_t lb = s.length / block_size;
      const int64_t off = s.length % block_size;
      if (lb == static_cast<int64_t>(s.blocks.size())) {
        s.blocks.push_back(pop_gpu());
      } else if (gpu.ref[static_cast<size_t>(s.blocks[static_cast<size_t>(lb)])] > 1) {
        const int32_t src = s.blocks[static_cast<size_t>(lb)];
        const int32_t dst = pop_gpu();
        --gpu.ref[static_cast<size_t>(src)];
        s.blocks[static_cast<size_t>(lb)] = dst;
        if (pairs) {
          pairs[2 * np] = src;
          pairs[2 * np + 1] = dst;
        }
        ++np;
        ++st.cow_copies;
      }
      if (slots) slots[t] = static_cast<int64_t>(s.blocks[static_cast<size_t>(lb)]) * block_size + off;
      ++s.length;
    }
    if (npairs) *npairs = np;
  }

  int32_t request_state(int64_t r) const { return seqs.at(requests.at(r).front()).state; }

  std::vector<int32_t> distinct_blocks(int64_t r) const {
    std::vector<int32_t> order;
    std::unordered_set<int32_t> seen;
    for (int64_t sid : requests.at(r))
      for (int32_t b : seqs.at(sid).blocks)
        if (seen.insert(b).second) order.push_back(b);
    return order;
  }
};

extern "C" {

const char* pa_bm_last_error(void) { return g_bm_error.c_str(); }

pa_bm* pa_bm_create(int32_t num_blocks, int32_t num_cpu_blocks, int32_t block_size,
                    const int32_t* free_order, const int32_t* cpu_free_order) {
  if (num_blocks <= 0 || num_cpu_blocks < 0 || block_size <= 0) {
    bm_fail(PA_BM_INVALID, "pa_bm_create: num_blocks and block_size must be positive");
    return nullptr;
  }
  pa_bm* bm = new (std::nothrow) pa_bm();
  if (!bm) {
    bm_fail(PA_BM_INVALID, "pa_bm_create: out of host memory");
    return nullptr;
  }
  bm->block_size = block_size;
  if (!bm->gpu.init(num_blocks, free_order) || !bm->cpu.init(num_cpu_blocks, cpu_free_order)) {
    delete bm;
    bm_fail(PA_BM_INVALID, "pa_bm_create: a free order is not a permutation of the block ids");
    return nullptr;
  }
  bm->st.num_blocks = num_blocks;
  bm->st.num_cpu_blocks = num_cpu_blocks;
  bm_ok();
  return bm;
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

pa_bm_status pa_bm_add_sequence(pa_bm* bm, int64_t seq_id, int64_t num_tokens,
                                int64_t* slots_out) {
  if (!bm || num_tokens < 0) return bm_fail(PA_BM_INVALID, "pa_bm_add_sequence: bad argument");
  if (bm->seqs.count(seq_id))
    return bm_fail(PA_BM_INVALID, "pa_bm_add_sequence: sequence %lld already exists",
                   static_cast<long long>(seq_id));
  const int64_t need = bm->blocks_for(num_tokens);
  if (need > bm->gpu.num_free()) {
    ++bm->st.allocation_failures;
    return bm_fail(PA_BM_OUT_OF_BLOCKS, "pa_bm_add_sequence: need %lld blocks, %d free",
                   static_cast<long long>(need), bm->gpu.num_free());
  }
  const int64_t r = bm->next_request++;
  bm->requests[r] = {seq_id};
  Seq& s = bm->seqs[seq_id];
  s.request = r;
  bm->append(s, num_tokens, slots_out, nullptr, nullptr);
  return bm_ok();
}

pa_bm_status pa_bm_append(pa_bm* bm, int64_t seq_id, int64_t num_new, int64_t* slots_out,
                          int64_t* cow_pairs_out, int32_t cow_capacity, int32_t* num_cow) {
  if (!bm || num_new < 0) return bm_fail(PA_BM_INVALID, "pa_bm_append: bad argument");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return bm_fail(PA_BM_INVALID, "pa_bm_append: unknown sequence %lld",
                   static_cast<long long>(seq_id));
  Seq& s = it->second;
  if (s.state != PA_BM_RUNNING)
    return bm_fail(PA_BM_WRONG_STATE, "pa_bm_append: sequence %lld is preempted",
                   static_cast<long long>(seq_id));
  const int64_t need = bm->blocks_needed(s, num_new);
  const bool may_copy = num_new > 0 && !s.blocks.empty() &&
                        bm->gpu.ref[static_cast<size_t>(s.blocks.back())] > 1 &&
                        s.length % bm->block_size != 0;
  if (may_copy && (cow_capacity < 1 || !cow_pairs_out))
    return bm_fail(PA_BM_INVALID, "pa_bm_append: room for one copy pair is needed");
  if (need > bm->gpu.num_free()) {
    ++bm->st.allocation_failures;
    return bm_fail(PA_BM_OUT_OF_BLOCKS, "pa_bm_append: need %lld blocks, %d free",
                   static_cast<long long>(need), bm->gpu.num_free());
  }
  int32_t np = 0;
  bm->append(s, num_new, slots_out, cow_pairs_out, &np);
  if (num_cow) *num_cow = np;
  return bm_ok();
}

pa_bm_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child) {
  if (!bm) return bm_fail(PA_BM_INVALID, "pa_bm_fork: null manager");
  auto it = bm->seqs.find(parent);
  if (it == bm->seqs.end())
    return bm_fail(PA_BM_INVALID, "pa_bm_fork: unknown sequence %lld",
                   static_cast<long long>(parent));
  if (bm->seqs.count(child))
    return bm_fail(PA_BM_INVALID, "pa_bm_fork: sequence %lld already exists",
                   static_cast<long long>(child));
  if (it->second.state != PA_BM_RUNNING)
    return bm_fail(PA_BM_WRONG_STATE, "pa_bm_fork: parent %lld is preempted",
                   static_cast<long long>(parent));
  Seq c;
  c.blocks = it->second.blocks;
  c.length = it->second.length;
  c.request = it->second.request;
  for (int32_t b : c.blocks) ++bm->gpu.ref[static_cast<size_t>(b)];
  bm->requests[c.request].push_back(child);
  bm->seqs.emplace(child, std::move(c));
  return bm_ok();
}

pa_bm_status pa_bm_free(pa_bm* bm, int64_t seq_id) {
  if (!bm) return bm_fail(PA_BM_INVALID, "pa_bm_free: null manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return bm_fail(PA_BM_INVALID, "pa_bm_free: unknown sequence %lld",
                   static_cast<long long>(seq_id));
  Seq& s = it->second;
  for (int32_t b : s.blocks) {
    if (s.state == PA_BM_SWAPPED) {
      if (--bm->cpu.ref[static_cast<size_t>(b)] == 0) bm->cpu.free_stack.push_back(b);
    } else {
      bm->release_gpu(b);
    }
  }
  auto& members = bm->requests[s.request];
  members.erase(std::find(members.begin(), members.end(), seq_id));
  if (members.empty()) bm->requests.erase(s.request);
  bm->seqs.erase(it);
  return bm_ok();
}

int64_t pa_bm_blocks_needed(const pa_bm* bm, int64_t seq_id, int64_t num_new) {
  if (!bm || num_new < 0) return -1;
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end() || it->second.state != PA_BM_RUNNING) return -1;
  return bm->blocks_needed(it->second, num_new);
}

pa_bm_status pa_bm_seq_info(const pa_bm* bm, int64_t seq_id, int64_t* length,
                            int32_t* num_blocks, int32_t* state, int64_t* request,
                            int64_t* recompute_tokens) {
  if (!bm) return bm_fail(PA_BM_INVALID, "pa_bm_seq_info: null manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return bm_fail(PA_BM_INVALID, "pa_bm_seq_info: unknown sequence %lld",
                   static_cast<long long>(seq_id));
  const Seq& s = it->second;
  if (length) *length = s.length;
  if (num_blocks) *num_blocks = static_cast<int32_t>(s.blocks.size());
  if (state) *state = s.state;
  if (request) *request = s.request;
  if (recompute_tokens) *recompute_tokens = s.recompute_tokens;
  return bm_ok();
}

pa_bm_status pa_bm_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t capacity) {
  if (!bm) return bm_fail(PA_BM_INVALID, "pa_bm_table: null manager");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end())
    return bm_fail(PA_BM_INVALID, "pa_bm_table: unknown sequence %lld",
                   static_cast<long long>(seq_id));
  const auto& b = it->second.blocks;
  if (static_cast<int64_t>(b.size()) > capacity || (!out && !b.empty()))
    return bm_fail(PA_BM_INVALID, "pa_bm_table: capacity %d < %zu blocks", capacity, b.size());
  std::copy(b.begin(), b.end(), out);
  return bm_ok();
}

pa_bm_status pa_bm_block_tables(const pa_bm* bm, const int64_t* seq_ids, int32_t n,
                                int32_t width, int32_t* out) {
  if (!bm || n < 0 || width <= 0 || (n > 0 && (!seq_ids || !out)))
    return bm_fail(PA_BM_INVALID, "pa_bm_block_tables: bad argument");
  for (int32_t i = 0; i < n; ++i) {
    auto it = bm->seqs.find(seq_ids[i]);
    if (it == bm->seqs.end())
      return bm_fail(PA_BM_INVALID, "pa_bm_block_tables: unknown sequence %lld",
                     static_cast<long long>(seq_ids[i]));
    if (static_cast<int64_t>(it->second.blocks.size()) > width)
      return bm_fail(PA_BM_INVALID, "pa_bm_block_tables: width %d < %zu blocks", width,
                     it->second.blocks.size());
  }
  for (int32_t i = 0; i < n; ++i) {
    const auto& b = bm->seqs.at(seq_ids[i]).blocks;
    int32_t* row = out + static_cast<size_t>(i) * width;
    std::fill(row, row + width, -1);
    std::copy(b.begin(), b.end(), row);
  }
  return bm_ok();
}

int32_t pa_bm_refcount(const pa_bm* bm, int32_t block, int32_t on_cpu) {
  if (!bm) return -1;
  const Pool& p = on_cpu ? bm->cpu : bm->gpu;
  if (block < 0 || block >= static_cast<int32_t>(p.ref.size())) return -1;
  return p.ref[static_cast<size_t>(block)];
}

pa_bm_status pa_bm_preempt_latest(pa_bm* bm, int32_t mode, int64_t protect_request,
                                  int64_t* request_out, int64_t* pairs_out, int32_t capacity,
                                  int32_t* num_pairs) {
  if (!bm || (mode != PA_BM_MODE_SWAP && mode != PA_BM_MODE_RECOMPUTE))
    return bm_fail(PA_BM_INVALID, "pa_bm_preempt_latest: bad argument");
  int64_t victim = -1;
  for (auto it = bm->requests.rbegin(); it != bm->requests.rend(); ++it) {
    if (it->first != protect_request && bm->request_state(it->first) == PA_BM_RUNNING) {
      victim = it->first;
      break;
    }
  }
  if (victim < 0) return bm_fail(PA_BM_NO_VICTIM, "pa_bm_preempt_latest: no running request");
  if (mode == PA_BM_MODE_SWAP) {
    const std::vector<int32_t> blocks = bm->distinct_blocks(victim);
    const int32_t nb = static_cast<int32_t>(blocks.size());
    if (nb > bm->cpu.num_free())
      return bm_fail(PA_BM_OUT_OF_BLOCKS, "pa_bm_preempt_latest: swap needs %d CPU blocks, %d "
                     "free", nb, bm->cpu.num_free());
    if (nb > capacity || (nb > 0 && !pairs_out))
      return bm_fail(PA_BM_INVALID, "pa_bm_preempt_latest: room for %d pairs needed", nb);
    std::unordered_map<int32_t, int32_t> remap;
    for (int32_t i = 0; i < nb; ++i) {
      const int32_t g = blocks[static_cast<size_t>(i)];
      const int32_t c = bm->cpu.pop();
      bm->cpu.ref[static_cast<size_t>(c)] = bm->gpu.ref[static_cast<size_t>(g)];
      bm->gpu.ref[static_cast<size_t>(g)] = 0;
      bm->gpu.free_stack.push_back(g);
      ++bm->st.blocks_freed;
      remap[g] = c;
      pairs_out[2 * i] = g;
      pairs_out[2 * i + 1] = c;
    }
    for (int64_t sid : bm->requests[victim]) {
      Seq& s = bm->seqs.at(sid);
      for (auto& b : s.blocks) b = remap.at(b);
      s.state = PA_BM_SWAPPED;
    }
    ++bm->st.preemptions_swap;
    bm->st.blocks_swapped_out += nb;
    if (num_pairs) *num_pairs = nb;
  } else {
    for (int64_t sid : bm->requests[victim]) {
      Seq& s = bm->seqs.at(sid);
      for (int32_t b : s.blocks) bm->release_gpu(b);
      s.recompute_tokens = s.length;
      s.length = 0;
      s.blocks.clear();
      s.state = PA_BM_RECOMPUTE;
    }
    ++bm->st.preemptions_recompute;
    if (num_pairs) *num_pairs = 0;
  }
  if (request_out) *request_out = victim;
  return bm_ok();
}

pa_bm_status pa_bm_swap_in_earliest(pa_bm* bm, int64_t* request_out, int64_t* pairs_out,
                                    int32_t capacity, int32_t* num_pairs) {
  if (!bm) return bm_fail(PA_BM_INVALID, "pa_bm_swap_in_earliest: null manager");
  int64_t r = -1;
  for (const auto& kv : bm->requests) {
    if (bm->request_state(kv.first) == PA_BM_SWAPPED) {
      r = kv.first;
      break;
    }
  }
  if (r < 0) return bm_fail(PA_BM_NO_VICTIM, "pa_bm_swap_in_earliest: no swapped request");
  const std::vector<int32_t> blocks = bm->distinct_blocks(r);
  const int32_t nb = static_cast<int32_t>(blocks.size());
  if (nb > bm->gpu.num_free()) {
    ++bm->st.allocation_failures;
    return bm_fail(PA_BM_OUT_OF_BLOCKS, "pa_bm_swap_in_earliest: needs %d blocks, %d free", nb,
                   bm->gpu.num_free());
  }
  if (nb > capacity || (nb > 0 && !pairs_out))
    return bm_fail(PA_BM_INVALID, "pa_bm_swap_in_earliest: room for %d pairs needed", nb);
  std::unordered_map<int32_t, int32_t> remap;
  for (int32_t i = 0; i < nb; ++i) {
    const int32_t c = blocks[static_cast<size_t>(i)];
    const int32_t g = bm->pop_gpu();
    bm->gpu.ref[static_cast<size_t>(g)] = bm->cpu.ref[static_cast<size_t>(c)];
    bm->cpu.ref[static_cast<size_t>(c)] = 0;
    bm->cpu.free_stack.push_back(c);
    remap[c] = g;
    pairs_out[2 * i] = c;
    pairs_out[2 * i + 1] = g;
  }
  for (int64_t sid : bm->requests[r]) {
    Seq& s = bm->seqs.at(sid);
    for (auto& b : s.blocks) b = remap.at(b);
    s.state = PA_BM_RUNNING;
  }
  bm->st.blocks_swapped_in += nb;
  if (num_pairs) *num_pairs = nb;
  if (request_out) *request_out = r;
  return bm_ok();
}

pa_bm_status pa_bm_resume_recompute(pa_bm* bm, int64_t request) {
  if (!bm) return bm_fail(PA_BM_INVALID, "pa_bm_resume_recompute: null manager");
  auto it = bm->requests.find(request);
  if (it == bm->requests.end() || bm->request_state(request) != PA_BM_RECOMPUTE)
    return bm_fail(PA_BM_WRONG_STATE, "pa_bm_resume_recompute: request %lld is not waiting "
                   "for recompute", static_cast<long long>(request));
  for (int64_t sid : it->second) bm->seqs.at(sid).state = PA_BM_RUNNING;
  return bm_ok();
}

pa_bm_status pa_bm_request_members(const pa_bm* bm, int64_t request, int64_t* out,
                                   int32_t capacity, int32_t* count) {
  if (!bm) return bm_fail(PA_BM_INVALID, "pa_bm_request_members: null manager");
  auto it = bm->requests.find(request);
  if (it == bm->requests.end())
    return bm_fail(PA_BM_INVALID, "pa_bm_request_members: unknown request %lld",
                   static_cast<long long>(request));
  const auto& m = it->second;
  if (count) *count = static_cast<int32_t>(m.size());
  if (static_cast<int64_t>(m.size()) > capacity || (!out && !m.empty()))
    return bm_fail(PA_BM_INVALID, "pa_bm_request_members: capacity %d < %zu", capacity,
                   m.size());
  std::copy(m.begin(), m.end(), out);
  return bm_ok();
}

pa_bm_status pa_bm_get_stats(const pa_bm* bm, pa_bm_stats* out) {
  if (!bm || !out) return bm_fail(PA_BM_INVALID, "pa_bm_get_stats: bad argument");
  *out = bm->st;
  out->free_blocks = bm->gpu.num_free();
  out->free_cpu_blocks = bm->cpu.num_free();
  int64_t waste = 0;
  for (const auto& kv : bm->seqs) {
    const Seq& s = kv.second;
    if (s.state == PA_BM_RUNNING) waste += bm->blocks_for(s.length) * bm->block_size - s.length;
  }
  out->tail_waste_slots = waste;
  out->num_sequences = static_cast<int64_t>(bm->seqs.size());
  out->num_requests = static_cast<int64_t>(bm->requests.size());
  return bm_ok();
}

// ------------------------------------------------------------------- step planner (token cap)
// The rules are those of include/block_manager.h (pa_sp_*); step_planner.py states them in
// Python and the two are tested against each other.

}  // extern "C"

struct pa_sp {
  pa_bm* bm = nullptr;
  int32_t max_tokens = 0;
  int32_t max_chunk = 0;                                    // <= 0: no per-chunk limit
  std::vector<std::pair<int64_t, int64_t>> prefilling;      // (sequence, prompt tokens left)
  std::vector<int64_t> decoding;

  bool queued(int64_t seq) const {
    for (const auto& p : prefilling)
      if (p.first == seq) return true;
    return std::find(decoding.begin(), decoding.end(), seq) != decoding.end();
  }
};

extern "C" {

pa_sp* pa_sp_create(pa_bm* bm, int32_t max_tokens_per_step, int32_t max_chunk) {
  if (!bm || max_tokens_per_step <= 0 || max_chunk < 0) {
    bm_fail(PA_BM_INVALID, "pa_sp_create: need a manager, a positive cap and max_chunk >= 0");
    return nullptr;
  }
  pa_sp* sp = new (std::nothrow) pa_sp();
  if (!sp) {
    bm_fail(PA_BM_INVALID, "pa_sp_create: out of host memory");
    return nullptr;
  }
  sp->bm = bm;
  sp->max_tokens = max_tokens_per_step;
  sp->max_chunk = max_chunk;
  bm_ok();
  return sp;
}

void pa_sp_destroy(pa_sp* sp) { delete sp; }

pa_bm_status pa_sp_set_limits(pa_sp* sp, int32_t max_tokens_per_step, int32_t max_chunk) {
  if (!sp || max_tokens_per_step <= 0 || max_chunk < 0)
    return bm_fail(PA_BM_INVALID, "pa_sp_set_limits: need a positive cap and max_chunk >= 0");
  sp->max_tokens = max_tokens_per_step;
  sp->max_chunk = max_chunk;
  return bm_ok();
}

pa_bm_status pa_sp_add_request(pa_sp* sp, int64_t seq_id, int64_t prompt_len) {
  if (!sp || prompt_len <= 0)
    return bm_fail(PA_BM_INVALID, "pa_sp_add_request: a prompt holds at least one token");
  if (sp->queued(seq_id) || sp->bm->seqs.count(seq_id))
    return bm_fail(PA_BM_INVALID, "pa_sp_add_request: sequence %lld already exists",
                   static_cast<long long>(seq_id));
  sp->prefilling.emplace_back(seq_id, prompt_len);
  return bm_ok();
}

pa_bm_status pa_sp_finish(pa_sp* sp, int64_t seq_id) {
  if (!sp) return bm_fail(PA_BM_INVALID, "pa_sp_finish: null planner");
  auto it = std::find(sp->decoding.begin(), sp->decoding.end(), seq_id);
  if (it == sp->decoding.end())
    return bm_fail(PA_BM_WRONG_STATE, "pa_sp_finish: sequence %lld is not decoding",
                   static_cast<long long>(seq_id));
  const pa_bm_status st = pa_bm_free(sp->bm, seq_id);
  if (st != PA_BM_OK) return st;
  sp->decoding.erase(it);
  return bm_ok();
}

pa_bm_status pa_sp_counts(const pa_sp* sp, int32_t* num_decoding, int32_t* num_prefilling) {
  if (!sp) return bm_fail(PA_BM_INVALID, "pa_sp_counts: null planner");
  if (num_decoding) *num_decoding = static_cast<int32_t>(sp->decoding.size());
  if (num_prefilling) *num_prefilling = static_cast<int32_t>(sp->prefilling.size());
  return bm_ok();
}

pa_bm_status pa_sp_step(pa_sp* sp, pa_sp_plan* plan) {
  if (!sp || !plan) return bm_fail(PA_BM_INVALID, "pa_sp_step: bad argument");
  pa_bm* bm = sp->bm;
  const int64_t ndec = static_cast<int64_t>(sp->decoding.size());
  const int64_t npre = static_cast<int64_t>(sp->prefilling.size());
  const int64_t max_slots = std::max<int64_t>(ndec, sp->max_tokens);
  if (plan->decode_capacity < ndec || plan->chunk_capacity < npre ||
      plan->slot_capacity < max_slots || plan->cow_capacity < ndec + npre ||
      (ndec && !plan->decode_seqs) || (npre && (!plan->chunk_seqs || !plan->chunk_lens)) ||
      (max_slots && !plan->slot_mapping) || ((ndec + npre) && !plan->cow_pairs))
    return bm_fail(PA_BM_INVALID, "pa_sp_step: output capacities must cover %lld decodes, "
                   "%lld chunks, %lld slots and %lld copy pairs",
                   static_cast<long long>(ndec), static_cast<long long>(npre),
                   static_cast<long long>(max_slots), static_cast<long long>(ndec + npre));
  // the decodes' blocks first, all or nothing
  int64_t need = 0;
  for (int64_t sid : sp->decoding) {
    auto it = bm->seqs.find(sid);
    if (it == bm->seqs.end() || it->second.state != PA_BM_RUNNING)
      return bm_fail(PA_BM_WRONG_STATE, "pa_sp_step: decoding sequence %lld is not resident",
                     static_cast<long long>(sid));
    need += bm->blocks_needed(it->second, 1);
  }
  if (need > bm->gpu.num_free())
    return bm_fail(PA_BM_OUT_OF_BLOCKS, "pa_sp_step: the step's decodes need %lld blocks, %d "
                   "free", static_cast<long long>(need), bm->gpu.num_free());
  std::vector<int64_t> dec_slots(static_cast<size_t>(ndec));
  int32_t ncow = 0;
  for (int64_t i = 0; i < ndec; ++i) {
    const int64_t sid = sp->decoding[static_cast<size_t>(i)];
    int32_t np = 0;
    bm->append(bm->seqs.at(sid), 1, &dec_slots[static_cast<size_t>(i)],
               plan->cow_pairs + 2 * ncow, &np);
    plan->decode_seqs[i] = sid;
    ncow += np;
  }
  // then prompt chunks in arrival order, within what the cap leaves
  int64_t left = std::max<int64_t>(0, static_cast<int64_t>(sp->max_tokens) - ndec);
  int32_t nchunk = 0;
  int64_t nslot = 0;
  std::vector<size_t> done;
  for (size_t i = 0; i < sp->prefilling.size() && left > 0; ++i) {
    const int64_t sid = sp->prefilling[i].first;
    const int64_t rem = sp->prefilling[i].second;
    int64_t n = std::min(rem, left);
    if (sp->max_chunk > 0) n = std::min<int64_t>(n, sp->max_chunk);
    auto it = bm->seqs.find(sid);
    if (it != bm->seqs.end()) {
      if (it->second.state != PA_BM_RUNNING || bm->blocks_needed(it->second, n) > bm->gpu.num_free())
        break;
      int32_t np = 0;
      bm->append(it->second, n, plan->slot_mapping + nslot, plan->cow_pairs + 2 * ncow, &np);
      ncow += np;
    } else {
      if (bm->blocks_for(n) > bm->gpu.num_free()) break;
      const int64_t r = bm->next_request++;
      bm->requests[r] = {sid};
      Seq& s = bm->seqs[sid];
      s.request = r;
      bm->append(s, n, plan->slot_mapping + nslot, nullptr, nullptr);
    }
    plan->chunk_seqs[nchunk] = sid;
    plan->chunk_lens[nchunk] = n;
    ++nchunk;
    nslot += n;
    left -= n;
    if (n == rem) done.push_back(i);
    else sp->prefilling[i].second = rem - n;
  }
  for (auto d = done.rbegin(); d != done.rend(); ++d) {
    sp->decoding.push_back(sp->prefilling[*d].first);
    sp->prefilling.erase(sp->prefilling.begin() + static_cast<std::ptrdiff_t>(*d));
  }
  // finished prompts join the decodes in arrival order
  if (done.size() > 1)
    std::reverse(sp->decoding.end() - static_cast<std::ptrdiff_t>(done.size()), sp->decoding.end());
  std::copy(dec_slots.begin(), dec_slots.end(), plan->slot_mapping + nslot);
  plan->num_chunks = nchunk;
  plan->num_decodes = static_cast<int32_t>(ndec);
  plan->num_slots = static_cast<int32_t>(nslot + ndec);
  plan->num_cow = ncow;
  return bm_ok();
}

}  // extern "C"
