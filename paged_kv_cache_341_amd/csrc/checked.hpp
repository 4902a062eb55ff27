// Checked mode of the C ABI: host-side validation of the device-content preconditions (table
// entries, lengths, chunk offsets, slots, copy pairs, group plans) that the kernels rely on but
// do not check.  Off by default; on with the environment variable PA_CHECKED=1 or
// pa_set_checked_mode(1).  Each check copies the index arrays to the host on the caller's
// stream (so it sees the values the kernels would read) and synchronises that stream, so it
// costs a device round trip per call: a debugging aid, not for the hot path.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>

namespace pa {
namespace checked {

bool enabled();
bool set_enabled(bool on);   // returns the previous setting

// Each returns "" when the contents meet the preconditions, else a message naming the first
// violation (a failed copy is reported the same way).  tables() with block_tables == nullptr
// checks the lengths only.
std::string tables(hipStream_t st, const int32_t* block_tables, const int32_t* seq_lens,
                   int num_seqs, int max_blocks_per_seq, int num_blocks, int block_size,
                   int max_seq_len);
std::string chunks(hipStream_t st, const int32_t* query_start_loc, const int32_t* seq_lens,
                   int num_chunks, int total_q, int max_q_len);
std::string slots(hipStream_t st, const int64_t* slot_mapping, int num_tokens, int num_blocks,
                  int block_size);
// same_pool: source and destination are one pool (copy-on-write), so no destination may also
// be a source; otherwise (swap) the two id ranges are checked separately.
std::string pairs(hipStream_t st, const int64_t* block_pairs, int num_pairs, int num_src_blocks,
                  int num_dst_blocks, bool same_pool);
std::string groups(hipStream_t st, const int32_t* group_start, const int32_t* shared_blocks,
                   const int32_t* block_tables, const int32_t* seq_lens, int num_seqs,
                   int num_groups, int max_group_size, int max_blocks_per_seq, int block_size);

}  // namespace checked
}  // namespace pa
