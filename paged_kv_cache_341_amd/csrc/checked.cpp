// Checked mode: host-side validation of device-content preconditions (see checked.hpp).
#include "checked.hpp"

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <unordered_set>
#include <vector>

namespace pa {
namespace checked {

namespace {

// -1: not yet read from the environment
std::atomic<int> g_mode{-1};

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  snprintf(buf, sizeof(buf), f, a, b, c);
  return buf;
}

// Copies n elements from device (or mapped host) memory, ordered after the work already on st.
template <typename T>
std::string fetch(hipStream_t st, const T* src, size_t n, std::vector<T>& dst) {
  dst.resize(n);
  if (n == 0) return "";
  hipError_t e = hipMemcpyAsync(dst.data(), src, n * sizeof(T), hipMemcpyDefault, st);
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  if (e != hipSuccess) return std::string("copy of an index array failed: ") + hipGetErrorString(e);
  return "";
}

}  // namespace

bool enabled() {
  int m = g_mode.load(std::memory_order_relaxed);
  if (m < 0) {
    const char* e = std::getenv("PA_CHECKED");
    m = (e && e[0] && std::strcmp(e, "0") != 0) ? 1 : 0;
    int expected = -1;
    if (!g_mode.compare_exchange_strong(expected, m)) m = expected;
  }
  return m == 1;
}

bool set_enabled(bool on) {
  const bool prev = enabled();
  g_mode.store(on ? 1 : 0);
  return prev;
}

std::string tables(hipStream_t st, const int32_t* block_tables, const int32_t* seq_lens,
                   int num_seqs, int max_blocks_per_seq, int num_blocks, int block_size,
                   int max_seq_len) {
  std::vector<int32_t> sl, bt;
  std::string err = fetch(st, seq_lens, static_cast<size_t>(num_seqs), sl);
  if (err.empty() && block_tables)
    err = fetch(st, block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, bt);
  if (!err.empty()) return err;
  for (int s = 0; s < num_seqs; ++s) {
    const int L = sl[s];
    if (L < 1 || L > max_seq_len)
      return fmt("sequence %lld: seq_len %lld outside [1, max_seq_len %lld]", s, L, max_seq_len);
    if (!block_tables) continue;
    const int used = (L + block_size - 1) / block_size;
    for (int j = 0; j < used; ++j) {
      const int32_t b = bt[static_cast<size_t>(s) * max_blocks_per_seq + j];
      if (b < 0 || b >= num_blocks)
        return fmt("sequence %lld: table entry %lld holds block id %lld, outside the pool", s, j,
                   b);
    }
  }
  return "";
}

std::string chunks(hipStream_t st, const int32_t* query_start_loc, const int32_t* seq_lens,
                   int num_chunks, int total_q, int max_q_len) {
  std::vector<int32_t> qsl, sl;
  std::string err = fetch(st, query_start_loc, static_cast<size_t>(num_chunks) + 1, qsl);
  if (err.empty()) err = fetch(st, seq_lens, static_cast<size_t>(num_chunks), sl);
  if (!err.empty()) return err;
  if (qsl[0] != 0 || qsl[num_chunks] != total_q)
    return fmt("query_start_loc runs from %lld to %lld, not from 0 to total_q %lld", qsl[0],
               qsl[num_chunks], total_q);
  for (int c = 0; c < num_chunks; ++c) {
    const int n = qsl[c + 1] - qsl[c];
    if (n < 0) return fmt("query_start_loc falls at chunk %lld", c);
    if (n > max_q_len) return fmt("chunk %lld has %lld rows, more than max_q_len %lld", c, n,
                                  max_q_len);
    if (n > sl[c]) return fmt("chunk %lld has %lld rows, more than its seq_len %lld", c, n, sl[c]);
  }
  return "";
}

std::string slots(hipStream_t st, const int64_t* slot_mapping, int num_tokens, int num_blocks,
                  int block_size) {
  std::vector<int64_t> sm;
  std::string err = fetch(st, slot_mapping, static_cast<size_t>(num_tokens), sm);
  if (!err.empty()) return err;
  const int64_t limit = static_cast<int64_t>(num_blocks) * block_size;
  std::unordered_set<int64_t> seen;
  seen.reserve(sm.size() * 2);
  for (int t = 0; t < num_tokens; ++t) {
    const int64_t s = sm[t];
    if (s < 0) continue;                       // padding
    if (s >= limit) return fmt("token %lld: slot %lld outside the pool (%lld slots)", t, s, limit);
    if (!seen.insert(s).second) return fmt("token %lld: slot %lld is written twice", t, s);
  }
  return "";
}

std::string pairs(hipStream_t st, const int64_t* block_pairs, int num_pairs, int num_src_blocks,
                  int num_dst_blocks, bool same_pool) {
  std::vector<int64_t> p;
  std::string err = fetch(st, block_pairs, static_cast<size_t>(num_pairs) * 2, p);
  if (!err.empty()) return err;
  std::unordered_set<int64_t> dsts, srcs;
  for (int i = 0; i < num_pairs; ++i) {
    const int64_t src = p[2 * i], dst = p[2 * i + 1];
    if (src < 0 || src >= num_src_blocks)
      return fmt("pair %lld: source block %lld outside the pool", i, src);
    if (dst < 0 || dst >= num_dst_blocks)
      return fmt("pair %lld: destination block %lld outside the pool", i, dst);
    if (!dsts.insert(dst).second) return fmt("pair %lld: destination %lld appears twice", i, dst);
    srcs.insert(src);
  }
  if (same_pool)
    for (int i = 0; i < num_pairs; ++i)
      if (srcs.count(p[2 * i + 1]))
        return fmt("pair %lld: destination %lld is also a source", i, p[2 * i + 1]);
  return "";
}

std::string groups(hipStream_t st, const int32_t* group_start, const int32_t* shared_blocks,
                   const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                   int num_groups, int max_group_size, int max_blocks_per_seq, int block_size) {
  std::vector<int32_t> gs, sb, bt, sl;
  std::string err = fetch(st, group_start, static_cast<size_t>(num_groups) + 1, gs);
  if (err.empty()) err = fetch(st, shared_blocks, static_cast<size_t>(num_seqs), sb);
  if (err.empty()) err = fetch(st, seq_lens, static_cast<size_t>(num_seqs), sl);
  if (err.empty())
    err = fetch(st, block_tables, static_cast<size_t>(num_seqs) * max_blocks_per_seq, bt);
  if (!err.empty()) return err;
  if (gs[0] != 0 || gs[num_groups] != num_seqs)
    return fmt("group_start runs from %lld to %lld, not from 0 to num_seqs %lld", gs[0],
               gs[num_groups], num_seqs);
  for (int g = 0; g < num_groups; ++g) {
    const int a = gs[g], b = gs[g + 1];
    if (b <= a) return fmt("group %lld is empty or group_start falls", g);
    if (b - a > max_group_size)
      return fmt("group %lld has %lld members, more than max_group_size %lld", g, b - a,
                 max_group_size);
    const int n = sb[a];
    for (int s = a; s < b; ++s) {
      if (sb[s] != n) return fmt("group %lld: sequence %lld disagrees on shared_blocks", g, s);
      if (n < 0 || static_cast<int64_t>(n) * block_size > sl[s])
        return fmt("sequence %lld: %lld shared blocks are not full blocks of it", s, n);
      const int32_t* row = bt.data() + static_cast<size_t>(s) * max_blocks_per_seq;
      const int32_t* first = bt.data() + static_cast<size_t>(a) * max_blocks_per_seq;
      if (!std::equal(row, row + std::min(n, max_blocks_per_seq), first))
        return fmt("group %lld: sequence %lld's shared table entries differ", g, s);
    }
  }
  return "";
}

}  // namespace checked
}  // namespace pa
