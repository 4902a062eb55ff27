/*
 * pagedattn.h - C ABI of the paged KV-cache hot path for MI355X (gfx950).
 *
 * The operations follow the pages' statement of the problem:
 *   - KV lives in a pool of equal, fixed-size physical blocks; a sequence's tokens fill its
 *     logical blocks left to right and a per-sequence block table maps each logical block to a
 *     physical one, so token j of a sequence sits in physical block table[j / B] at offset
 *     j % B.  (study-docs "PagedAttention & Continuous Batching", section "Block tables";
 *     cloudmash "Batching and PagedAttention", section "PagedAttention", steps 1-2.)
 *   - Attention gathers K and V through that table instead of assuming one contiguous slab.
 *     (cloudmash "PagedAttention", step 4; llmdeepdive "7.8", section "Concept".)
 *   - A sequence grows into its current block and takes a fresh one when it fills.
 *     (study-docs "Block tables".)
 *   - Forked sequences share blocks; the first write into a shared block copies it.
 *     (study-docs "Copy-on-write"; cloudmash "Sharing blocks".)
 *   - A continuous-batching step mixes chunks of long prompts with single-token decodes.
 *     (cloudmash "Continuous batching"; llmdeepdive "Concept", continuous-batching paragraph.)
 *
 * Layout (every entry point):
 *   k_cache, v_cache : [num_blocks][num_kv_heads][block_size][head_dim], row-major, one tensor
 *                      per layer.  A (block, kv head) slab is block_size*head_dim contiguous
 *                      elements.
 *   q, out           : [rows][num_q_heads][head_dim], row-major.
 *   Query head h reads kv head h / (num_q_heads / num_kv_heads).
 *   Element type: all of q, out, k_cache, v_cache, k_new, v_new share `dtype`.  Scores,
 *   softmax and accumulation are fp32; bf16 outputs are rounded to nearest-even once.
 *   Block tables and lengths are int32, slot mappings and copy pairs int64.
 *
 * Ownership: the caller owns every buffer.  Device pointers must be device memory of the
 * current HIP device; `stream` is a hipStream_t (NULL = the default stream).  The library never
 * allocates or frees memory, keeps no pointer after returning, and holds no mutable global state
 * beyond the checked-mode switch below and pa_decode_noalloc's static scratch array, so calls
 * from several host threads are safe (pa_decode_noalloc's own sharing rule aside).  Every call
 * only enqueues work on `stream`: no host synchronisation, no device-to-host copy (except in
 * checked mode).
 *
 * Errors: host scalars and pointers are checked before anything is enqueued; a failed check
 * returns a non-zero status, enqueues nothing, and sets a per-thread message readable through
 * pa_last_error().  Device contents (table entries, lengths, slots) are preconditions, not
 * checked: table entries read must lie in [0, num_blocks), 1 <= seq_lens[i] <= max_seq_len,
 * non-negative slots must be distinct and below num_blocks*block_size, copy destinations must be
 * distinct and never a source.  Violating them is undefined behaviour.  In checked mode
 * (pa_set_checked_mode, or the environment variable PA_CHECKED=1) every call first copies its
 * index arrays to the host on `stream`, synchronises that stream, and returns
 * PA_ERR_INVALID_ARGUMENT, enqueuing nothing, on the first violated precondition.  No C++
 * exception crosses this interface.
 */
#ifndef PAGEDATTN_H_
#define PAGEDATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, non-positive size, misalignment, bad ratio */
  PA_ERR_UNSUPPORTED = 2,        /* a valid request the library has no kernel for */
  PA_ERR_WORKSPACE_TOO_SMALL = 3,
  PA_ERR_DEVICE = 4              /* the HIP runtime reported an error at launch */
} pa_status;

typedef enum pa_dtype { PA_DTYPE_F32 = 0, PA_DTYPE_BF16 = 1 } pa_dtype;

/*
 * pa_decode - one query token per sequence attends to all of its seq_lens[s] cached tokens,
 * gathered through its block table (cloudmash "PagedAttention" step 4; study-docs "Block
 * tables").  seq_lens count the token appended in the same step, so that token sees itself.
 *
 *   out          [num_seqs][num_q_heads][head_dim]   written
 *   q            [num_seqs][num_q_heads][head_dim]
 *   block_tables [num_seqs][max_blocks_per_seq] int32 (entries past ceil(len/B) never read)
 *   seq_lens     [num_seqs] int32
 *   max_seq_len  host upper bound of seq_lens; sizes the split grid (no device read-back)
 *   scale        multiplies q.k before the softmax; finite and > 0
 *   workspace    device scratch of at least pa_decode_workspace_size(...) bytes (may be NULL
 *                when that size is 0); contents need no initialisation
 *
 * Supported: head_dim in {64, 128, 256}; block_size in {1, 4, 8, 16, 32, 64} (16 is the
 * pages' default; the others serve the block-size trade-off of cloudmash "Batching and
 * PagedAttention", section "Choosing the block size"); num_q_heads/num_kv_heads in
 * {1, 2, 4, 8}; dtype F32 or BF16.  Pointers 16-byte aligned.
 */
pa_status pa_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_blocks,
                    int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                    pa_dtype dtype, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of workspace pa_decode needs for these sizes (0 when no split is needed).  Besides the
 * sizes of the problem statement it takes num_kv_heads: the split plan sizes a split from the
 * number of (sequence, kv head) work items, so the number of partials depends on it. */
size_t pa_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                int32_t head_dim, int32_t block_size, int32_t max_seq_len);

/*
 * pa_decode_contiguous - the same decode over KV stored without paging: every (sequence, kv
 * head) owns one contiguous slab of `capacity` token rows, as in a cache that reserves room for
 * a maximum length up front.  It is pa_decode with the block-table lookup taken out (same split
 * and merge, same unit of 16 tokens as 16-token blocks), the contiguous baseline that the
 * pages weigh paging against: attention through a block table is slower than over one
 * contiguous slab (cloudmash "Batching and PagedAttention", section "The indirection has a
 * cost").  Result: as pa_decode on the same rows (up to fp32 summation order).
 *
 *   out, q       [num_seqs][num_q_heads][head_dim]
 *   k, v         [num_seqs][num_kv_heads][capacity][head_dim]; row j < seq_lens[s] of
 *                (s, kv head) is token j; rows past it are never used
 *   seq_lens     [num_seqs] int32, 1 <= seq_lens[s] <= max_seq_len
 *   capacity     token rows per (sequence, kv head): a multiple of 16, >= max_seq_len
 *   workspace    pa_decode_workspace_size(num_seqs, num_q_heads, num_kv_heads, head_dim, 16,
 *                max_seq_len) bytes; contents need no initialisation
 *
 * Supported as pa_decode.  Errors as pa_decode, plus PA_ERR_INVALID_ARGUMENT for a capacity
 * that is not a multiple of 16 or is below max_seq_len.
 */
pa_status pa_decode_contiguous(void* out, const void* q, const void* k, const void* v,
                               const int32_t* seq_lens, int32_t num_seqs, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t capacity,
                               int32_t max_seq_len, float scale, pa_dtype dtype,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * pa_decode_noalloc - for callers that cannot allocate device memory: code under HIP graph
 * capture, serving loops and harnesses that forbid allocation.  Same arguments (less the
 * workspace) and the same result, bit for bit, as pa_decode, on the same kernels; the split
 * partials go to a static device array inside the library instead of a caller workspace.
 *
 *   Scratch: PA_DECODE_NOALLOC_SCRATCH_BYTES per GPU, held from the first call on that GPU until
 *            the process ends.  The call allocates and frees nothing.
 *   Limit:   sizes with pa_decode_workspace_size(...) > PA_DECODE_NOALLOC_SCRATCH_BYTES are
 *            refused with PA_ERR_WORKSPACE_TOO_SMALL before anything is enqueued.
 *   Sharing: every call on one GPU uses that GPU's array, which keeps the last call's partials;
 *            calls that overlap on one GPU (other streams, other host threads) race and give
 *            undefined results.  `stream` must belong to the current device.
 *   Errors:  those of pa_decode, and PA_ERR_DEVICE if the array's address cannot be obtained on
 *            the current device.
 */
#define PA_DECODE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
pa_status pa_decode_noalloc(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                            int32_t head_dim, int32_t block_size, int32_t num_blocks,
                            int32_t max_blocks_per_seq, int32_t max_seq_len, float scale,
                            pa_dtype dtype, void* stream);

/*
 * pa_decode_grouped - pa_decode for a batch whose sequences come in groups that share a
 * prefix of physical blocks: parallel samples or beams forked from one prompt hold the same
 * blocks until a write forces a copy (study-docs "PagedAttention & Continuous Batching",
 * section "Copy-on-write"; cloudmash "Batching and PagedAttention", section "Sharing blocks").
 * The result equals pa_decode's on the same arguments (up to fp32 summation order); the shared
 * blocks are read once per group instead of once per member, and the group's query rows attend
 * to them together on MFMA.
 *
 *   group_start   [num_groups+1] int32, rising from 0 to num_seqs: group g is the sequences
 *                 group_start[g] .. group_start[g+1]-1 (a group of one is allowed)
 *   shared_blocks [num_seqs] int32: the number of leading blocks the sequence shares with its
 *                 group; equal within a group, and table entries 0 .. shared_blocks-1 equal
 *                 within a group (only the group's first table is read for them).  Clamped
 *                 on the device to 0 .. floor(seq_lens/block_size): only full blocks are shared.
 *   max_group_size host upper bound of group sizes
 *   other arguments as pa_decode; workspace of pa_decode_grouped_workspace_size(...) bytes,
 *   contents need no initialisation
 *
 * Supported: dtype BF16, head_dim 64, 128 or 256, block_size 16, num_q_heads/num_kv_heads in
 * {1, 2, 4, 8}.  Arguments that break the equalities above give wrong values, never an
 * access outside the buffers the other arguments describe.
 */
pa_status pa_decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_tables, const int32_t* seq_lens,
                            const int32_t* group_start, const int32_t* shared_blocks,
                            int32_t num_seqs, int32_t num_groups, int32_t max_group_size,
                            int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                            int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                            int32_t max_seq_len, float scale, pa_dtype dtype, void* workspace,
                            size_t workspace_bytes, void* stream);

/* Bytes of workspace pa_decode_grouped needs for these sizes (0 for unsupported sizes). */
size_t pa_decode_grouped_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                        int32_t num_kv_heads, int32_t head_dim,
                                        int32_t block_size, int32_t max_seq_len);

/*
 * pa_prefill_chunk - attention for chunks of new prompt tokens over a paged prefix
 * (cloudmash "Continuous batching": long prompts are processed in chunks across steps).
 * Chunk c owns packed query rows query_start_loc[c] .. query_start_loc[c+1]-1; its sequence
 * holds seq_lens[c] tokens after the chunk was appended, so row i of an n-row chunk sits at
 * position seq_lens[c]-n+i and sees keys 0 .. seq_lens[c]-n+i: the whole prefix, and the chunk
 * causally.  A one-row chunk is a decode.
 *
 *   out, q          [total_q][num_q_heads][head_dim]
 *   block_tables    [num_chunks][max_blocks_per_seq] int32
 *   seq_lens        [num_chunks] int32, each >= the chunk's row count
 *   query_start_loc [num_chunks+1] int32, rising from 0 to total_q
 *   max_q_len       host upper bound of the rows in one chunk
 *   max_seq_len     host upper bound of seq_lens
 *   scale           multiplies q.k before the softmax; finite and > 0
 *
 * Supported: dtype BF16 (MFMA bf16 -> fp32), head_dim 64, 128 or 256, block_size 16,
 * num_q_heads/num_kv_heads in {1, 2, 4, 8}.  Needs no workspace.  Up to 128 chunks are
 * scheduled longest first (ranked on the device from seq_lens); more are taken in order.
 */
pa_status pa_prefill_chunk(void* out, const void* q, const void* k_cache, const void* v_cache,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           const int32_t* query_start_loc, int32_t num_chunks, int32_t total_q,
                           int32_t max_q_len, int32_t max_seq_len, int32_t num_q_heads,
                           int32_t num_kv_heads, int32_t head_dim, int32_t block_size,
                           int32_t num_blocks, int32_t max_blocks_per_seq, float scale,
                           pa_dtype dtype, void* workspace, size_t workspace_bytes,
                           void* stream);

/* Bytes of workspace pa_prefill_chunk needs (currently always 0). */
size_t pa_prefill_workspace_size(int32_t num_chunks, int32_t total_q, int32_t num_q_heads,
                                 int32_t head_dim, int32_t max_seq_len);

/*
 * kv_append - write new tokens' K and V rows into their slots (study-docs "Block tables": a
 * sequence grows into its current block).  For each t with slot_mapping[t] >= 0:
 *   k_cache[slot / block_size][:][slot % block_size][:] = k_new[t][:][:]   (same for V)
 * as an exact bit copy.  Negative slots are padding and are skipped.
 *
 *   k_new, v_new  [num_tokens][num_kv_heads][head_dim]
 *   slot_mapping  [num_tokens] int64, slot = physical_block * block_size + offset
 *
 * Supported: head_dim a multiple of 16 bytes' worth of elements, block_size 16 (any positive
 * block_size is accepted), F32 or BF16.  num_tokens == 0 is a no-op.
 */
pa_status kv_append(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                    const int64_t* slot_mapping, int32_t num_tokens, int32_t num_kv_heads,
                    int32_t head_dim, int32_t block_size, int32_t num_blocks, pa_dtype dtype,
                    void* stream);

/*
 * cow_copy_blocks - copy-on-write block copies (study-docs "Copy-on-write": a write into a
 * shared block first takes a fresh block and copies the old one into it).  For each pair p:
 *   k_cache[pairs[p][1]] = k_cache[pairs[p][0]]; v_cache[pairs[p][1]] = v_cache[pairs[p][0]]
 * whole blocks (every kv head, every slot), as exact bit copies.
 *
 *   block_pairs  [num_pairs][2] int64 (src, dst); num_pairs == 0 is a no-op
 */
pa_status cow_copy_blocks(void* k_cache, void* v_cache, const int64_t* block_pairs,
                          int32_t num_pairs, int32_t num_kv_heads, int32_t head_dim,
                          int32_t block_size, int32_t num_blocks, pa_dtype dtype, void* stream);

/*
 * pa_mixed_step - one continuous-batching iteration's attention work in a single persistent
 * launch: the KV append of the iteration's new tokens, then the chunked-prefill rows and the
 * decode rows together (cloudmash "Batching and PagedAttention", section "Continuous
 * batching": prompt chunks and decode steps share an iteration, long prompts cut into chunks;
 * llmdeepdive "Concept", continuous-batching paragraph).  Results equal kv_append followed by
 * pa_prefill_chunk on the chunk fields and pa_decode on the decode fields (up to fp32
 * summation order in the decodes).  Chunk rows are bound by the matrix cores and decode rows
 * by HBM; one kernel runs both at once, one workgroup per CU, each taking work from a queue of
 * chunk tiles (longest chunk first) and a queue of decode splits.  Enqueues three launches
 * (append, the mixed kernel, the decode merge), no host synchronisation.
 *
 * Fields (pa_mixed_batch): the append's k_new, v_new [num_new_tokens][num_kv_heads][head_dim]
 * and slot_mapping (as kv_append; num_new_tokens may be 0); the chunks' out, q, tables,
 * seq_lens, query_start_loc and host bounds (as pa_prefill_chunk; num_chunks may be 0); the
 * decodes' out, q, tables, seq_lens and host bounds (as pa_decode; num_seqs may be 0); the pool
 * and head counts shared by both.  Workspace: pa_mixed_workspace_size(...) bytes, contents need
 * no initialisation; the call uses its first 256 bytes as work counters and the rest as the
 * decode split partials.
 *
 * Supported: dtype BF16, head_dim 64, 128 or 256, block_size 16, num_q_heads/num_kv_heads in
 * {1, 2, 4, 8}, at most 128 chunks and 2048 decode sequences.  Device-content preconditions
 * are those of the three calls it replaces.
 */
typedef struct pa_mixed_batch {
  /* append */
  const void* k_new;
  const void* v_new;
  const int64_t* slot_mapping;
  int32_t num_new_tokens;
  /* chunked prefill */
  void* chunk_out;
  const void* chunk_q;
  const int32_t* chunk_tables;
  const int32_t* chunk_seq_lens;
  const int32_t* query_start_loc;
  int32_t num_chunks, chunk_total_q, chunk_max_q_len, chunk_max_seq_len;
  int32_t chunk_max_blocks_per_seq;
  /* decode */
  void* dec_out;
  const void* dec_q;
  const int32_t* dec_tables;
  const int32_t* dec_seq_lens;
  int32_t num_seqs, dec_max_seq_len, dec_max_blocks_per_seq;
  /* pool */
  void* k_cache;
  void* v_cache;
  int32_t num_q_heads, num_kv_heads, head_dim, block_size, num_blocks;
  float scale;
  pa_dtype dtype;
} pa_mixed_batch;

pa_status pa_mixed_step(const pa_mixed_batch* batch, void* workspace, size_t workspace_bytes,
                        void* stream);

/* Bytes of workspace pa_mixed_step needs (0 for unsupported sizes). */
size_t pa_mixed_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t block_size, int32_t dec_max_seq_len);

/*
 * swap_blocks - whole-block copies between two pools, for preemption by swapping: every block
 * of a preempted request moves to the host pool at once, and back to the device when the
 * request resumes (cloudmash "Batching and PagedAttention", section "When blocks run out").  For each
 * pair p:
 *   dst_k[pairs[p][1]] = src_k[pairs[p][0]]; dst_v[pairs[p][1]] = src_v[pairs[p][0]]
 * whole blocks, exact bit copies.  Both pools have the layout of the device pool
 * ([blocks][num_kv_heads][block_size][head_dim]); either may be host memory that the device
 * can map (pinned with hipHostMalloc), the other device memory: swap-out copies device to host,
 * swap-in host to device.  The pairs come from pa_bm_preempt_latest / pa_bm_swap_in_earliest
 * (block_manager.h) and live in device or mapped host memory.
 *
 *   block_pairs  [num_pairs][2] int64 (src block, dst block); num_pairs == 0 is a no-op
 *
 * Preconditions (not checked on the device; checks.check_swap_pairs checks them on the host):
 * src ids in [0, num_src_blocks), dst ids in [0, num_dst_blocks), dst ids distinct.  The
 * source and destination pools must be different allocations.
 */
pa_status swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                      const int64_t* block_pairs, int32_t num_pairs, int32_t num_kv_heads,
                      int32_t head_dim, int32_t block_size, int32_t num_src_blocks,
                      int32_t num_dst_blocks, pa_dtype dtype, void* stream);

/*
 * pa_hbm_read_probe - a diagnostic, not part of the paged path: reads `bytes` of device memory
 * at `src` with 16-byte non-temporal loads (the load the decode kernel streams KV with) on
 * `num_workgroups` workgroups of 256 lanes, and writes one XOR-folded word per lane to `sink`
 * (num_workgroups * 256 uint32, device).  Timing it gives the achievable HBM read rate that
 * decode bandwidth is compared against.  bytes: a positive multiple of 16; src 16-byte aligned;
 * num_workgroups in [1, 2^20].
 */
pa_status pa_hbm_read_probe(const void* src, size_t bytes, uint32_t* sink,
                            int32_t num_workgroups, void* stream);

/*
 * pa_mfma_probe - a diagnostic, not part of the paged path: on `num_workgroups` workgroups of 512
 * lanes, every wave runs `iters` rounds of four independent bf16 32x32x16 matrix-core
 * accumulations on register operands (2 * 32 * 32 * 16 * 4 * iters flops per wave, no memory
 * traffic) and writes one value per lane to `sink` (num_workgroups * 512 floats, device).
 * Timing it gives the achievable dense bf16 MFMA rate that prefill is compared against.
 * num_workgroups in [1, 2^20], iters > 0.
 */
pa_status pa_mfma_probe(float* sink, int32_t num_workgroups, int32_t iters, void* stream);

/* Static, human-readable name of a status code. */
const char* pa_status_string(pa_status s);

/* Per-thread description of the last failed call on this thread ("" if none). */
const char* pa_last_error(void);

/*
 * Checked mode, for callers that cannot trust their index arrays (debugging, untrusted input):
 * when on, pa_decode, pa_decode_grouped, pa_prefill_chunk, pa_mixed_step, kv_append,
 * cow_copy_blocks and swap_blocks validate their device-content preconditions on host copies
 * (table entries used, seq_lens in [1, max_seq_len], query_start_loc rising from 0 to total_q
 * with chunks no longer than max_q_len or their sequence, slots in range and distinct, copy
 * pairs in range with distinct destinations that are never a source, group plans as
 * pa_decode_grouped requires) before enqueuing anything.  Each such call synchronises its
 * stream once.  Process-wide; off unless PA_CHECKED is set to a value other than "0".
 * pa_set_checked_mode returns the previous setting (0 or 1); pa_checked_mode the current one.
 */
int pa_set_checked_mode(int enable);
int pa_checked_mode(void);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDATTN_H_ */
