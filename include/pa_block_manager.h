/*
 * pa_block_manager.h -- host-side block manager for the paged KV cache of
 * libpa: the producer of the block tables, lengths and write slots that the
 * kernels in pa.h consume.  Pure host code; no call touches the GPU.
 *
 * What it manages follows the pages' description of dynamic memory
 * management ("vLLM's efficiency secret: PagedAttention and dynamic memory
 * management", section "Dynamic memory management": a BlockSpaceManager with
 * a pool of GPU blocks of block_size tokens and CPU blocks, which checks
 * whether a new request can be admitted before allocating its blocks):
 *   - a request of n tokens needs ceil(n / block_size) blocks; it is admitted
 *     only if that many blocks are free, else nothing changes
 *     (PA_ERR_OUT_OF_BLOCKS);
 *   - blocks are handed out as a request grows and returned as soon as it is
 *     freed ("Efficient Memory Management ... paper summary", key feature 4);
 *   - requests may share blocks (key feature 2, block-level sharing): a fork
 *     gives a new request the blocks of an existing one;
 *   - the usage ratio is the share of GPU blocks in use (the deployment tip's
 *     block_usage_ratio).
 * Readings where the pages are silent: shared blocks carry reference counts
 * and are freed when the count reaches zero; a request about to write into a
 * partly filled shared block first gets a private copy of it (copy-on-write:
 * the call reports the (source, destination) block pair to copy, e.g. with
 * pa_copy_blocks); free blocks are handed out lowest id first; swapping moves
 * a request's blocks between GPU and CPU one for one and is refused for
 * requests that share blocks.
 *
 * Sequence ids are any non-negative ints chosen by the caller.  Block ids are
 * indices into the GPU pool (or the CPU pool for swapped-out requests).
 * A manager is not thread-safe: calls on one manager must not overlap.
 * Errors return a pa_status (pa.h) and leave the manager unchanged; the
 * detail is in pa_last_error().
 */
#ifndef PA_BLOCK_MANAGER_H_
#define PA_BLOCK_MANAGER_H_

#include <stdint.h>

#include "pa.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_bm pa_bm;

/* A manager for num_gpu_blocks GPU blocks and num_cpu_blocks CPU blocks of
 * block_size tokens each (block_size >= 1, num_gpu_blocks >= 1,
 * num_cpu_blocks >= 0).  *out receives the new manager. */
int pa_bm_create(int block_size, int num_gpu_blocks, int num_cpu_blocks, pa_bm** out);

/* Release a manager (NULL is ignored). */
void pa_bm_destroy(pa_bm* bm);

/* 1 if a request of num_tokens tokens can be admitted now, 0 if not, or a
 * negative -pa_status for invalid arguments. */
int pa_bm_can_allocate(const pa_bm* bm, int num_tokens);

/* Admit sequence seq_id holding num_tokens tokens (its prompt): it gets
 * ceil(num_tokens / block_size) GPU blocks.  PA_ERR_OUT_OF_BLOCKS if too few
 * are free; PA_ERR_INVALID_ARG if seq_id exists or num_tokens < 0. */
int pa_bm_allocate(pa_bm* bm, int seq_id, int num_tokens);

/* Make room for one more token of seq_id.  *slot_block / *slot_row receive
 * where the new token goes (the position context_lens - 1 of the decode
 * calls once the length counts it).  If the last block was full a new block
 * is added; if it is partly filled and shared, it is replaced by a private
 * copy and *cow_src / *cow_dst receive the blocks to copy (else both -1).
 * Any output pointer may be NULL. */
int pa_bm_append_slot(pa_bm* bm, int seq_id, int32_t* slot_block, int32_t* slot_row,
                      int32_t* cow_src, int32_t* cow_dst);

/* New sequence child_id sharing all blocks of parent_id (same length). */
int pa_bm_fork(pa_bm* bm, int parent_id, int child_id);

/* Drop seq_id; its blocks whose reference count reaches zero become free. */
int pa_bm_free(pa_bm* bm, int seq_id);

/* Move seq_id's blocks to the CPU (swap_out) or back (swap_in).  pairs
 * receives (source block, destination block) for each of its blocks, in
 * table order, at most max_pairs pairs (PA_ERR_INVALID_ARG if more are
 * needed); *num_pairs receives the count. */
int pa_bm_swap_out(pa_bm* bm, int seq_id, int32_t* pairs, int max_pairs, int* num_pairs);
int pa_bm_swap_in(pa_bm* bm, int seq_id, int32_t* pairs, int max_pairs, int* num_pairs);

/* Free GPU (on_cpu = 0) or CPU (on_cpu = 1) blocks, or -pa_status. */
int pa_bm_num_free_blocks(const pa_bm* bm, int on_cpu);

/* Share of GPU blocks in use, in [0, 1] (negative for a NULL manager). */
double pa_bm_usage_ratio(const pa_bm* bm);

/* Length, block count and location (0 GPU, 1 CPU) of seq_id. */
int pa_bm_seq_info(const pa_bm* bm, int seq_id, int* num_tokens, int* num_blocks, int* on_cpu);

/* Reference count of a GPU or CPU block, or -pa_status. */
int pa_bm_refcount(const pa_bm* bm, int block, int on_cpu);

/* The rows of a decode batch: for i < n, block_tables[i][0..nb) = the GPU
 * blocks of seq_ids[i] (nb <= max_blocks_per_seq, the rest filled with -1)
 * and context_lens[i] = its length.  Every listed sequence must be on the
 * GPU. */
int pa_bm_fill_batch(const pa_bm* bm, const int32_t* seq_ids, int n, int32_t* block_tables,
                     int max_blocks_per_seq, int32_t* context_lens);

/* Prompt groups of a decode batch, for pa_decode_shared_prefix: sequences
 * whose first full block is the same physical block form a group, whose
 * shared prompt is the longest run of leading blocks full in, and identical
 * across, all members.  seq_group[i] receives the group of seq_ids[i] or -1;
 * group_prefix_len[j] the prompt tokens of group j (groups numbered in order
 * of first appearance, at most n / 2 of them); *num_groups and
 * *max_group_size receive the counts. */
int pa_bm_prefix_groups(const pa_bm* bm, const int32_t* seq_ids, int n, int32_t* seq_group,
                        int32_t* group_prefix_len, int* num_groups, int* max_group_size);

#ifdef __cplusplus
}
#endif

#endif /* PA_BLOCK_MANAGER_H_ */
