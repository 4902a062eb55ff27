/*
 * block_manager.h - native host-side allocator for a paged KV pool (C ABI).
 *
 * What it manages, as the pages describe it:
 *   - a pool of equal physical blocks (16 tokens by default); each sequence sees logical
 *     blocks filled left to right and a block table maps them to physical blocks; blocks are
 *     taken one at a time as the current one fills and a finished sequence returns them
 *     (cloudmash "Batching and PagedAttention", section "PagedAttention", steps 1-3;
 *     study-docs "PagedAttention & Continuous Batching", section "Block tables");
 *   - fork shares the parent's block ids and raises their reference counts; the first write
 *     into a shared block takes a fresh block and copies (study-docs "Copy-on-write";
 *     cloudmash "Sharing blocks");
 *   - on exhaustion, preemption takes the newest request first and moves all of its blocks
 *     at once: they go to the host pool, or they are dropped and the request's tokens are
 *     run again later (cloudmash, "When blocks run out");
 *   - capacity is counted in blocks so admission can refuse early, and the manager keeps the
 *     counters the pages name: free and used blocks, allocation failures, tail waste,
 *     preemptions (llmdeepdive "PagedAttention & continuous batching", section "Concept").
 *
 * Readings where the pages are silent (the Python BlockManager in block_manager.py follows
 * the same ones; the two are tested against each other):
 *   - a writer that finds a block's count above one copies it; the last holder writes in
 *     place;
 *   - a request is a sequence admitted with pa_bm_add_sequence plus all of its forks;
 *     arrival order is admission order; preemption evicts a whole request;
 *   - swap-out gives each distinct GPU block of the request one CPU block (members in request
 *     order, blocks in table order, first appearance) and carries its reference count;
 *     swap-in mirrors it and takes the earliest-arrived swapped request first;
 *   - recompute frees the blocks and keeps each member's token count; after
 *     pa_bm_resume_recompute each member re-appends its tokens into private blocks;
 *   - free stacks: freed blocks are reused first; the initial order is given by the caller.
 *
 * Slots are block * block_size + offset (int64).  Copy pairs are (src, dst) block ids:
 * copy-on-write pairs within the GPU pool, swap-out pairs (gpu, cpu), swap-in pairs
 * (cpu, gpu); the caller runs them on the device (cow_copy_blocks, swap_blocks) before the
 * blocks they free are written.
 *
 * Threading: a pa_bm is not thread-safe; calls on different managers are independent.  On
 * failure a call changes nothing, returns a non-zero status and leaves a message for
 * pa_bm_last_error on the calling thread.  No call allocates device memory or touches a GPU.
 */
#ifndef PAGED_KV_BLOCK_MANAGER_H_
#define PAGED_KV_BLOCK_MANAGER_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm;

typedef enum pa_bm_status {
  PA_BM_OK = 0,
  PA_BM_INVALID = 1,          /* bad argument: size, unknown or duplicate id, output too small */
  PA_BM_OUT_OF_BLOCKS = 2,    /* the pool (or the CPU pool for a swap) is short */
  PA_BM_NO_VICTIM = 3,        /* nothing to preempt or to swap in */
  PA_BM_WRONG_STATE = 4       /* the sequence or request is not in the state the call needs */
} pa_bm_status;

typedef enum pa_bm_seq_state { PA_BM_RUNNING = 0, PA_BM_SWAPPED = 1, PA_BM_RECOMPUTE = 2 } pa_bm_seq_state;
typedef enum pa_bm_mode { PA_BM_MODE_SWAP = 0, PA_BM_MODE_RECOMPUTE = 1 } pa_bm_mode;

typedef struct pa_bm_stats {
  int64_t num_blocks, free_blocks, num_cpu_blocks, free_cpu_blocks;
  int64_t allocation_failures, cow_copies, blocks_allocated, blocks_freed;
  int64_t preemptions_swap, preemptions_recompute, blocks_swapped_out, blocks_swapped_in;
  int64_t tail_waste_slots;   /* unfilled slots in the last blocks of GPU-resident sequences */
  int64_t num_sequences, num_requests;
} pa_bm_stats;

/* A manager over num_blocks GPU blocks and num_cpu_blocks CPU blocks (may be 0).  The free
 * orders list the ids handed out first (index 0 first); NULL means 0, 1, 2, ...  Returns NULL
 * on a bad argument (see pa_bm_last_error). */
pa_bm* pa_bm_create(int32_t num_blocks, int32_t num_cpu_blocks, int32_t block_size,
                    const int32_t* free_order, const int32_t* cpu_free_order);
void pa_bm_destroy(pa_bm* bm);

/* Admit a new sequence (a new request) holding num_tokens tokens; slots_out (may be NULL)
 * receives their num_tokens slots.  OUT_OF_BLOCKS refuses it up front. */
pa_bm_status pa_bm_add_sequence(pa_bm* bm, int64_t seq_id, int64_t num_tokens,
                                int64_t* slots_out);

/* Grow a resident sequence by num_new tokens: slots_out (may be NULL) receives num_new slots,
 * cow_pairs_out receives num_cow (src, dst) pairs, at most cow_capacity (one suffices: only the
 * block being written can be shared). */
pa_bm_status pa_bm_append(pa_bm* bm, int64_t seq_id, int64_t num_new, int64_t* slots_out,
                          int64_t* cow_pairs_out, int32_t cow_capacity, int32_t* num_cow);

pa_bm_status pa_bm_fork(pa_bm* bm, int64_t parent, int64_t child);
pa_bm_status pa_bm_free(pa_bm* bm, int64_t seq_id);

/* Free GPU blocks an append of num_new tokens would take (new blocks plus a copy), or -1. */
int64_t pa_bm_blocks_needed(const pa_bm* bm, int64_t seq_id, int64_t num_new);

/* length, number of blocks, state, request id and tokens awaiting recompute (NULLs allowed) */
pa_bm_status pa_bm_seq_info(const pa_bm* bm, int64_t seq_id, int64_t* length,
                            int32_t* num_blocks, int32_t* state, int64_t* request,
                            int64_t* recompute_tokens);

/* The sequence's block ids (CPU ids while swapped) into out[capacity]. */
pa_bm_status pa_bm_table(const pa_bm* bm, int64_t seq_id, int32_t* out, int32_t capacity);

/* int32 [n][width] tables of the given sequences, -1 past each one's blocks. */
pa_bm_status pa_bm_block_tables(const pa_bm* bm, const int64_t* seq_ids, int32_t n,
                                int32_t width, int32_t* out);

/* Reference count of a GPU (on_cpu = 0) or CPU block; -1 for an id out of range. */
int32_t pa_bm_refcount(const pa_bm* bm, int32_t block, int32_t on_cpu);

/* Preempt the most recently arrived running request other than `protect_request` (-1: none).
 * SWAP: pairs_out receives (gpu, cpu) pairs, num_pairs of them (capacity: at most the
 * request's block count).  RECOMPUTE: no pairs.  NO_VICTIM if there is none; OUT_OF_BLOCKS
 * (nothing changed) if the CPU pool cannot take the swap; INVALID if capacity is short. */
pa_bm_status pa_bm_preempt_latest(pa_bm* bm, int32_t mode, int64_t protect_request,
                                  int64_t* request_out, int64_t* pairs_out, int32_t capacity,
                                  int32_t* num_pairs);

/* Swap the earliest-arrived swapped request back in: (cpu, gpu) pairs. */
pa_bm_status pa_bm_swap_in_earliest(pa_bm* bm, int64_t* request_out, int64_t* pairs_out,
                                    int32_t capacity, int32_t* num_pairs);

/* Make a recompute-preempted request resident (empty); its members' token counts stay readable
 * through pa_bm_seq_info until they are re-appended by the caller. */
pa_bm_status pa_bm_resume_recompute(pa_bm* bm, int64_t request);

/* Members of a request, in request order, into out[capacity]; *count receives their number. */
pa_bm_status pa_bm_request_members(const pa_bm* bm, int64_t request, int64_t* out,
                                   int32_t capacity, int32_t* count);

pa_bm_status pa_bm_get_stats(const pa_bm* bm, pa_bm_stats* out);
const char* pa_bm_last_error(void);

/*
 * Step planner: one continuous-batching iteration at a time under a cap on the tokens a step
 * processes.  After every step finished sequences leave and waiting prompts join; long prompts
 * are cut into chunks spread over several steps (cloudmash "Batching and PagedAttention",
 * section "Continuous batching"; llmdeepdive "Concept", continuous-batching paragraph).  The cap
 * bounds how much prefill one step absorbs, which keeps the time per output token of decoding
 * requests steady, and requests are served first come, first served (cloudmash, section
 * "Scheduling is a policy, not just a mechanism"; llmdeepdive "Concept": maximum batch tokens).
 *
 * Readings where the pages are silent:
 *   - every decoding sequence runs in every step, one token each; prompts share what is left,
 *     max(0, cap - decodes) tokens;
 *   - prefilling requests take tokens in arrival order, each min(its prompt tokens left, the
 *     step's tokens left, max_chunk when max_chunk > 0); the rest of a prompt carries to the
 *     next step; a request that cannot get blocks for its chunk ends the step's prefill (no
 *     later arrival overtakes it); a prompt whose last chunk ran decodes from the next step on,
 *     queued after the decodes already running, in arrival order;
 *   - decodes take their blocks first, all or nothing: if the free blocks cannot cover every
 *     decode's append (counted per sequence), pa_sp_step returns PA_BM_OUT_OF_BLOCKS and changes
 *     nothing; making room (preemption) is the caller's decision;
 *   - the step's slot mapping lists the chunks' tokens in chunk order, then one token per
 *     decode in decode order: the layout kv_append and pa_mixed_step consume.
 * The planner drives `bm` (pa_bm_add_sequence on a prompt's first chunk, appends after that);
 * `bm` must outlive it, and the planner's sequences must not be changed through `bm` directly.
 */
typedef struct pa_sp pa_sp;

/* Outputs of pa_sp_step, in caller-owned arrays with their capacities.  Needed capacities:
 * decodes >= decoding sequences, chunks >= prefilling requests, slots >= max(decoding
 * sequences, cap), copy pairs >= decoding + prefilling (each append copies at most one block);
 * see pa_sp_counts.  chunk_lens are token counts; cow_pairs are (src, dst) block ids to copy on
 * the device (cow_copy_blocks) before the slots are written. */
typedef struct pa_sp_plan {
  int64_t* chunk_seqs;
  int64_t* chunk_lens;
  int32_t chunk_capacity, num_chunks;
  int64_t* decode_seqs;
  int32_t decode_capacity, num_decodes;
  int64_t* slot_mapping;
  int32_t slot_capacity, num_slots;
  int64_t* cow_pairs;          /* [capacity][2] */
  int32_t cow_capacity, num_cow;
} pa_sp_plan;

/* A planner over `bm` with a cap of max_tokens_per_step tokens per step (> 0) and at most
 * max_chunk prompt tokens per request per step (0: no limit).  NULL on a bad argument. */
pa_sp* pa_sp_create(pa_bm* bm, int32_t max_tokens_per_step, int32_t max_chunk);
void pa_sp_destroy(pa_sp* sp);

/* Change the cap and the per-request chunk limit from the next step on (same rules as
 * pa_sp_create). */
pa_bm_status pa_sp_set_limits(pa_sp* sp, int32_t max_tokens_per_step, int32_t max_chunk);

/* Queue a new prompt of prompt_len (> 0) tokens; its sequence must not exist yet. */
pa_bm_status pa_sp_add_request(pa_sp* sp, int64_t seq_id, int64_t prompt_len);

/* A decoding sequence is done: it leaves the batch and its blocks are freed. */
pa_bm_status pa_sp_finish(pa_sp* sp, int64_t seq_id);

/* Numbers of decoding sequences and of prefilling requests (NULLs allowed). */
pa_bm_status pa_sp_counts(const pa_sp* sp, int32_t* num_decoding, int32_t* num_prefilling);

/* Plan and allocate one step (rules above).  INVALID (nothing changed) if a capacity is short;
 * OUT_OF_BLOCKS (nothing changed) if the decodes' blocks do not fit. */
pa_bm_status pa_sp_step(pa_sp* sp, pa_sp_plan* plan);

#ifdef __cplusplus
}
#endif

#endif  /* PAGED_KV_BLOCK_MANAGER_H_ */
