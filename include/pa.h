/*
 * pa.h -- C ABI of libpa: paged KV-cache decode attention on AMD MI355X (gfx950).
 *
 * The data model follows the pages' description of paged KV caching:
 *   - the KV cache is one pool of fixed-size blocks ("pages"), each holding the
 *     keys (or values) of `block_size` consecutive tokens
 *     ("IO-5 vLLM Paged Attention", section 3 "KV Cache Paging structure";
 *      "Efficient Memory Management for LLM Serving with PagedAttention (vLLM)
 *      paper summary", key feature 1 "KV cache blocking");
 *   - each sequence owns a block table listing, in logical order, the physical
 *     blocks that hold its tokens, so its memory need not be contiguous
 *     ("IO-5 vLLM Paged Attention", section 2 "Paged Attention idea");
 *   - decode attention is softmax(q K^T * scale) V, with K and V the
 *     sequence's blocks concatenated in table order
 *     ("IO-5 vLLM Paged Attention", section 4 "Attention computation").
 *
 * Layouts (all row-major, element type `dtype`):
 *   q, out        [num_seqs][num_heads][head_dim]
 *   k_new, v_new  [num_seqs][num_kv_heads][head_dim]
 *   k_pool,v_pool [num_blocks][num_kv_heads][block_size][head_dim]
 *   block_tables  int32 [num_seqs][max_blocks_per_seq]
 *   context_lens  int32 [num_seqs]
 * Token t of sequence s, KV head g, lives at
 *   pool[block_tables[s][t / block_size]][g][t % block_size][:].
 * Query head h reads KV head h / (num_heads / num_kv_heads).
 *
 * Ownership and execution: every pointer argument is a DEVICE pointer owned by
 * the caller (except pa_check_inputs_host, which takes HOST pointers).  The
 * library allocates nothing and keeps no caller pointer after a call returns
 * (pa_decode_splitk_noalloc works in a static array of the library's own).
 * Every call only enqueues work on `stream` (a hipStream_t passed as void*;
 * NULL = the null stream) and returns without synchronising.  Calls are
 * thread-safe; the only global state is the calling thread's last-error
 * string, the per-device address of that static array, and the array.
 *
 * Errors: the host-side scalar checks below run before anything is enqueued; a
 * failing call returns a nonzero pa_status, enqueues nothing and records a
 * message for pa_last_error().  Device data (lengths, table entries) are not
 * read by the host.  If they break the contract, the kernels do not read or
 * write outside the buffers: an out-of-range length or block id makes that
 * sequence's output NaN (decode) or skips that sequence's write (cache write).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PA_ABI_VERSION 1

typedef enum {
  PA_F32 = 0,
  PA_F16 = 1,
  PA_BF16 = 2
} pa_dtype;

typedef enum {
  PA_OK = 0,
  PA_ERR_NULL = 1,          /* a required pointer is NULL */
  PA_ERR_INVALID_ARG = 2,   /* a size or relation between sizes is invalid */
  PA_ERR_UNSUPPORTED = 3,   /* head_dim, block_size or dtype not built */
  PA_ERR_WORKSPACE = 4,     /* split-K workspace missing or too small */
  PA_ERR_HIP = 5,           /* the HIP runtime reported an error on launch */
  PA_ERR_OUT_OF_BLOCKS = 6  /* block manager: too few free blocks, nothing changed */
} pa_status;

/* Decode flag bits.
 * PA_FLAG_SHARED_KV: some blocks are named by more than one sequence's table
 *   in this call (for example a prompt shared by parallel samples, block-level
 *   sharing as in "Efficient Memory Management ... paper summary", key feature
 *   2).  K/V loads then go through the caches normally so that later readers
 *   of a shared block can hit.  Without it every K/V load carries the
 *   non-temporal hint: each block is read once per call and would only
 *   displace other cache lines.  The flag changes speed, never results. */
#define PA_FLAG_SHARED_KV 1
/* PA_FLAG_VALU_ONLY: compute grouped query heads (num_heads > num_kv_heads,
 *   fp16/bf16) on the vector ALUs instead of the matrix cores.  Both paths
 *   accumulate in fp32 and meet the same error bounds; their results may
 *   differ in the last bits.  Meant for cross-checks and measurement. */
#define PA_FLAG_VALU_ONLY 2

/* Supported shapes: head_dim in {64, 128}; block_size a power of two in
 * [1, 65536] (a block at least as long as a sequence's largest length gives
 * the contiguous per-sequence cache as a special case); num_heads a multiple
 * of num_kv_heads; dtype one of pa_dtype. */

/* Version of this ABI (PA_ABI_VERSION of the built library). */
int pa_abi_version(void);

/* Static text for a pa_status value. */
const char* pa_status_str(int status);

/* Detail of the calling thread's last failed call ("" if none). */
const char* pa_last_error(void);

/*
 * pa_cache_write -- store each sequence's newest token into its block.
 *
 * The pages have a sequence's K/V stored block by block through its table
 * ("IO-5 vLLM Paged Attention", sections 2-3) and blocks handed out on demand
 * ("Efficient Memory Management ... paper summary", key feature 4); the write
 * of the token being decoded is not described there.  Reading used here:
 * context_lens[s] already counts the new token, which is logical position
 * L-1 with L = context_lens[s]; the caller has already placed a block in the
 * table for that position.  For every sequence with L >= 1 and every KV head
 * g the head_dim elements of k_new[s][g] and v_new[s][g] are copied, bit for
 * bit, to row (L-1) % block_size of block block_tables[s][(L-1)/block_size]
 * of k_pool and v_pool.  L = 0 writes nothing.  No other byte changes.
 * Two sequences must not name the same slot (undefined which write wins).
 *
 * num_seqs == 0 is a no-op (pointers may then be NULL).
 */
int pa_cache_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                   const int32_t* block_tables, const int32_t* context_lens,
                   int num_seqs, int num_kv_heads, int head_dim, int block_size,
                   int max_blocks_per_seq, int num_blocks, int dtype, void* stream);

/*
 * pa_decode -- single-pass paged decode attention.
 *
 * out[s][h] = softmax(q[s][h] . K_s^T * scale) V_s, where K_s, V_s are the
 * first L = context_lens[s] rows of KV head h / (num_heads/num_kv_heads) of
 * the blocks block_tables[s][0 .. ceil(L/block_size)-1] concatenated in order
 * ("IO-5 vLLM Paged Attention", section 4 "Attention computation"; block
 * count as in "vLLM's efficiency secret: PagedAttention and dynamic memory
 * management", section "Dynamic memory management").  Rows past L and table
 * entries past ceil(L/block_size) are never read and may hold anything.
 * Products and sums are accumulated in fp32; the result is rounded once to
 * `dtype` (nearest-even).  L = 0 gives a zero row.  `scale` is usually
 * 1/sqrt(head_dim).  `out` must not overlap any input.
 *
 * `flags` is a combination of PA_FLAG_SHARED_KV and PA_FLAG_VALU_ONLY;
 * other bits are rejected.
 *
 * One launch; no workspace.  Device contract: 0 <= L <= max_blocks_per_seq *
 * block_size and 0 <= block_tables[s][i] < num_blocks for i < ceil(L/bs);
 * a sequence that breaks it gets a NaN output row.
 */
int pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* context_lens,
              int num_seqs, int num_heads, int num_kv_heads, int head_dim,
              int block_size, int max_blocks_per_seq, int num_blocks,
              float scale, int dtype, int flags, void* stream);

/*
 * Bytes of device workspace pa_decode_splitk needs for these sizes: fp32
 * partial results for num_seqs * num_heads * ceil(max_context_len /
 * partition_size) partitions, each head_dim accumulators plus a running
 * maximum and sum, then the launch plan (256 bytes of counts, one 32-byte
 * unit record per possible (sequence, partition) pair, and 8 bytes per
 * sequence for the list of sequences with several partitions), each part
 * rounded up to 256 bytes.  Returns 0 for invalid sizes.
 */
size_t pa_decode_splitk_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                        int max_context_len, int partition_size);

/*
 * pa_decode_splitk -- the same result as pa_decode, computed in three
 * launches for long contexts: each sequence's L tokens are cut into
 * ceil(L / partition_size) partitions of equal length, rounded up to whole
 * 16-token steps, the last holding the rest (so none exceeds
 * `partition_size`, a positive multiple of 16).  A one-workgroup
 * planning launch lists the (sequence, partition) pairs longest first; the
 * partition launch takes them in that order and computes, per (sequence,
 * head, partition), the partition's maximum score m, sum of exp(score - m)
 * and unnormalised weighted value sum into `workspace`; the last launch
 * merges the partitions of each (sequence, head) of the sequences the plan
 * listed as split, in fixed order, rescaling each by exp(m_p - max_p m_p),
 * and writes `out`.  Sequences with a single partition are written directly
 * by the partition launch.  The result does
 * not depend on the order in which partitions run.
 *
 * max_context_len is a host-known bound on every context_lens[s] (no device
 * to host copy is made); it must not exceed max_blocks_per_seq * block_size.
 * It sizes the grid at ceil(max_context_len / partition_size) partitions
 * per sequence: a sequence that needs more gets a NaN output row (a longer
 * one that still fits them is computed normally).  `workspace` must hold
 * pa_decode_splitk_workspace_bytes(...) bytes, 16-byte aligned; its contents
 * on entry do not matter and are undefined on exit.
 */
int pa_decode_splitk(void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* context_lens,
                     int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                     int block_size, int max_blocks_per_seq, int num_blocks,
                     float scale, int dtype, int partition_size, int max_context_len,
                     void* workspace, size_t workspace_bytes, int flags, void* stream);

/* Size of the library's static device scratch used by pa_decode_splitk_noalloc. */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

/*
 * pa_decode_splitk_noalloc -- pa_decode_splitk for callers that cannot
 * allocate device memory: code under HIP graph capture, serving loops that
 * must not call the allocator, harnesses that forbid it.  Same arguments,
 * same kernels and the same result bits as pa_decode_splitk, but no
 * workspace argument: the split-K partials and the launch plan live in a
 * static device array of PA_NOALLOC_SCRATCH_BYTES (32 MiB) that the library
 * holds on each GPU it runs on until the process ends.  The call allocates
 * nothing (no hipMalloc, no hipFree, no allocating library routine); on its
 * first call on a device, with that device current, it looks up the array's
 * device address once and keeps it.
 *
 * Sizes whose workspace (pa_decode_splitk_workspace_bytes) exceeds
 * PA_NOALLOC_SCRATCH_BYTES are rejected with PA_ERR_WORKSPACE and a message
 * naming both sizes; nothing is launched.  PA_ERR_HIP if the scratch address
 * cannot be obtained.  All calls on one GPU share that GPU's scratch, which
 * keeps whatever the last call left (no call needs it cleared): calls that
 * may overlap on one GPU -- on different streams, or from different threads
 * -- race and must be ordered by the caller.
 */
int pa_decode_splitk_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int num_blocks,
                             float scale, int dtype, int partition_size, int max_context_len,
                             int flags, void* stream);

/*
 * Bytes of device workspace pa_decode_shared_prefix needs: the split-K
 * partials for ceil(max_context_len / partition_size) + 1 partitions per
 * sequence, the launch plan (its unit records also cover every group's
 * prompt partitions), and the group tables (a 16-byte member record and 8
 * bytes of plan scratch per sequence, 12 bytes per group).  Returns 0 for
 * invalid sizes.
 */
size_t pa_decode_shared_prefix_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                               int max_context_len, int partition_size,
                                               int num_groups);

/*
 * pa_decode_shared_prefix -- the same result as pa_decode for a batch in
 * which groups of sequences share the blocks of a common prompt (parallel
 * sampling, beam candidates): several requests using the same KV blocks is
 * the block-level sharing of "Efficient Memory Management ... paper summary",
 * key feature 2 and "Benefits" (less duplication of the KV cache).  Here the
 * sharing also saves bandwidth: each partition of a group's prompt is read
 * once, by one workgroup per KV head whose matrix-core columns are the
 * queries of every member, instead of once per member.
 *
 * seq_group[s] is the group of sequence s, or -1 for a sequence that shares
 * nothing; group_prefix_len[i] is the number of prompt tokens group i shares:
 * a multiple of block_size, at most every member's length, and the first
 * group_prefix_len[i] / block_size entries of every member's table name the
 * same blocks.  Each group has at most max_group_size members.
 *
 * Work units: the prompt is cut into partitions of partition_size tokens,
 * each computed once for all members.  A member's own tokens
 * [group_prefix_len, L) are absorbed into the group's last prompt partition
 * when there are at most partition_size / m of them, m being the most
 * members whose query columns share one chunk of 16 (16 / G for G query
 * heads per KV head dividing 16); that partition then streams each absorbed
 * member's tokens too, seen only by that member's columns, so it never
 * holds more than 2 * partition_size tokens.  Other members' own tokens,
 * and ungrouped sequences, are cut into partitions of their own, balanced
 * as in pa_decode_splitk.  A member
 * whose only partition is the absorbing one gets its output written
 * directly; otherwise partials are merged in fixed order as in
 * pa_decode_splitk.  Results are deterministic: the plan sorts each group's
 * members by sequence index.  A member's bits may depend on the lengths of
 * the members sorted before it in its chunk (which wave takes which of its
 * absorbed steps), not on their K/V values as long as those are finite.
 * A group that breaks the contract gives its members NaN rows.
 *
 * fp16 and bf16 only (PA_ERR_UNSUPPORTED otherwise); PA_FLAG_VALU_ONLY is
 * rejected.  PA_FLAG_SHARED_KV (cached loads) pays only when one prompt
 * partition is read by several column chunks, i.e. when a group has more
 * than 16 query columns (members * G); otherwise each prompt block is read
 * once per KV head and streaming loads (no flag) are faster.
 * max_context_len, partition_size and the workspace are as for
 * pa_decode_splitk, with pa_decode_shared_prefix_workspace_bytes(...) bytes.
 */
int pa_decode_shared_prefix(void* out, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* seq_group, const int32_t* group_prefix_len,
                            int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                            int dtype, int num_groups, int max_group_size, int partition_size,
                            int max_context_len, void* workspace, size_t workspace_bytes,
                            int flags, void* stream);

/*
 * pa_write_decode, pa_write_decode_splitk, pa_write_decode_shared_prefix --
 * one decode step in one call: pa_cache_write of each sequence's new token,
 * then pa_decode (resp. pa_decode_splitk, pa_decode_shared_prefix) over the
 * updated pools.
 * The pages store a sequence's K/V block by block through its table and
 * compute attention over the gathered blocks ("IO-5 vLLM Paged Attention",
 * sections 2-4); the new token's write is the reading stated at
 * pa_cache_write (position context_lens[s]-1, which the decode then
 * attends to).  The pools and `out` end with exactly the bytes the two
 * separate calls, in that order on one stream, would give.
 *
 * Why a combined call: one launch fewer per step.  The split-K plan reads
 * only the lengths (and groups), the write only the lengths, tables and new
 * rows, so the write runs in the plan's launch.  The single pass has no plan
 * launch; on the vector-ALU kernel (one query head per workgroup: MHA, or
 * fp32 with an odd group) over blocks of 16 tokens or more without
 * PA_FLAG_SHARED_KV, the decode launch itself stores the new rows and reads
 * row L-1 from k_new / v_new (the same bytes); in every other case
 * pa_write_decode launches the write and then the decode.
 *
 * Arguments: those of pa_decode (resp. pa_decode_splitk,
 * pa_decode_shared_prefix), with k_pool and v_pool written, plus k_new and
 * v_new ([num_seqs][num_kv_heads][head_dim], 16-byte aligned) as for
 * pa_cache_write.  k_new and v_new must not overlap the pools, `out` or the
 * workspace.  The slot a sequence's new token goes to must not be among the
 * rows any other sequence of the call attends to (a block that receives a
 * token belongs to one sequence, as copy-on-write ensures).  Every check of
 * both calls applies; if one fails nothing is launched.  num_seqs == 0 is a
 * no-op.
 */
int pa_write_decode(void* out, const void* q, void* k_pool, void* v_pool, const void* k_new,
                    const void* v_new, const int32_t* block_tables,
                    const int32_t* context_lens, int num_seqs, int num_heads,
                    int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                    int num_blocks, float scale, int dtype, int flags, void* stream);
int pa_write_decode_splitk(void* out, const void* q, void* k_pool, void* v_pool,
                           const void* k_new, const void* v_new,
                           const int32_t* block_tables, const int32_t* context_lens,
                           int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                           int block_size, int max_blocks_per_seq, int num_blocks,
                           float scale, int dtype, int partition_size, int max_context_len,
                           void* workspace, size_t workspace_bytes, int flags, void* stream);
int pa_write_decode_shared_prefix(void* out, const void* q, void* k_pool, void* v_pool,
                                  const void* k_new, const void* v_new,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* seq_group, const int32_t* group_prefix_len,
                                  int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_blocks_per_seq, int num_blocks,
                                  float scale, int dtype, int num_groups, int max_group_size,
                                  int partition_size, int max_context_len, void* workspace,
                                  size_t workspace_bytes, int flags, void* stream);

/*
 * pa_decode_contiguous -- the same decode attention over a contiguous KV
 * cache: the scheme paging replaces, in which every request reserves room for
 * the longest context it may reach ("IO-5 vLLM Paged Attention", section 1,
 * the contiguous KV problem; "vLLM's efficiency secret: PagedAttention and
 * dynamic memory management", section "KV cache like virtual memory", whose
 * example reserves the maximum context for every request).  It is here to
 * measure what the block-table indirection costs:
 * the kernels are those of pa_decode and pa_decode_splitk with the table
 * lookup removed, so for the same rows the result is the same bits as the
 * paged call (paging does not change the attention: "IO-5 vLLM Paged
 * Attention", "5 common misconceptions").
 *
 * k_cache and v_cache are [num_seqs][num_kv_heads][max_len][head_dim]: row t
 * of KV head g of sequence s is k_cache[s][g][t].  out[s][h] =
 * softmax(q[s][h] . K_s^T * scale) V_s over rows 0 .. L-1, L =
 * context_lens[s]; rows past L are never read and may hold anything.
 * Accumulation, rounding, L = 0 and the NaN row for 0 <= L <= max_len
 * broken are as for pa_decode.  max_len * head_dim * element size must not
 * exceed 2^31 - 1 bytes.
 *
 * partition_size 0: one pass, as pa_decode; `workspace` is not used (may be
 * NULL).  Otherwise the split-K launches of pa_decode_splitk with
 * max_context_len = max_len and a workspace of
 * pa_decode_splitk_workspace_bytes(num_seqs, num_heads, head_dim, max_len,
 * partition_size) bytes.  `flags`: 0 or PA_FLAG_VALU_ONLY (a contiguous
 * cache holds no shared rows, so PA_FLAG_SHARED_KV is rejected).
 */
int pa_decode_contiguous(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* context_lens, int num_seqs, int num_heads,
                         int num_kv_heads, int head_dim, int max_len, float scale, int dtype,
                         int partition_size, void* workspace, size_t workspace_bytes, int flags,
                         void* stream);

/*
 * pa_cache_write_contiguous -- pa_cache_write for the contiguous cache of
 * pa_decode_contiguous: for every sequence with 1 <= L <= max_len
 * (L = context_lens[s], which already counts the new token) and every KV
 * head g, the head_dim elements of k_new[s][g] and v_new[s][g] are copied,
 * bit for bit, to row L-1 of k_cache[s][g] and v_cache[s][g]
 * ([num_seqs][num_kv_heads][max_len][head_dim]).  Other lengths write
 * nothing; no other byte changes.  num_seqs == 0 is a no-op.
 */
int pa_cache_write_contiguous(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                              const int32_t* context_lens, int num_seqs, int num_kv_heads,
                              int head_dim, int max_len, int dtype, void* stream);

/*
 * pa_copy_blocks -- copy whole blocks of both pools, every KV head:
 * for i < num_pairs, block pairs[i][1] of k_pool and v_pool receives the
 * bytes of block pairs[i][0].  This is the private copy a shared, partly
 * filled block gets before a request writes into it (block-level sharing,
 * "Efficient Memory Management ... paper summary", key feature 2; the
 * copy-on-write reading of pa_block_manager.h).  `pairs` is a DEVICE array
 * int32 [num_pairs][2] (at most 65535 pairs).  Pairs naming a block outside
 * [0, num_blocks) are skipped; destinations must be distinct and must not be
 * sources of other pairs in the same call.  Asynchronous on `stream`.
 */
int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype,
                   void* stream);

/*
 * pa_swap_blocks -- move blocks between a device pool and a host pool (the
 * CPU blocks of "vLLM's efficiency secret ...", section "Dynamic memory
 * management", num_cpu_blocks): for i < num_pairs, block pairs[i][1] of
 * (dst_k, dst_v) receives block pairs[i][0] of (src_k, src_v), each block
 * `block_bytes` long.  to_host = 1 copies device -> host, 0 host -> device.
 * `pairs` is a HOST array int32 [num_pairs][2], checked against the pool
 * sizes (PA_ERR_INVALID_ARG).  Runs of consecutive pairs become one copy per
 * pool.  When the pairs form more than 8 runs of under 4 MiB each, and the
 * host pool is pinned memory with a device mapping (hipHostGetDevicePointer
 * succeeds, as for hipHostMalloc'd memory), one kernel per 256 pairs moves
 * the blocks through that mapping instead; block_bytes must then be a
 * multiple of 16 (else the copies are used).  Host pools should be pinned
 * for either form to be asynchronous on `stream`.
 */
int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                   const int32_t* pairs, int num_pairs, int num_dst_blocks, int num_src_blocks,
                   size_t block_bytes, int to_host, void* stream);

/*
 * pa_read_probe -- a measurement aid, not part of decode: reads num_tiles
 * tiles of tile_bytes bytes (a positive multiple of 4096) of the DEVICE
 * buffer `buf`, tile tile_order[i] at byte offset tile_order[i] * tile_bytes,
 * with the 16-byte non-temporal loads the decode kernels use, and writes
 * nothing (`sink`, a DEVICE uint32, is written only for one value the data
 * never produces).  tile_order (DEVICE int32 [num_tiles]) must name tiles
 * inside the buffer.  With an identity order it measures a sequential read;
 * with a random permutation of 4 KiB tiles, the scattered (block, head)
 * tiles of a paged pool: the read ceiling a decode kernel can approach on
 * this GPU.  Asynchronous on `stream`.
 */
int pa_read_probe(const void* buf, size_t tile_bytes, const int32_t* tile_order, int num_tiles,
                  uint32_t* sink, void* stream);

/*
 * pa_device_memory -- a measurement aid: the memory bus width in bits and the
 * peak memory clock in kHz that the HIP runtime reports for `device`, written
 * to *bus_width_bits and *mem_clock_khz (HOST ints).  Returns PA_ERR_NULL for a
 * NULL output pointer, PA_ERR_HIP (with the runtime's message in
 * pa_last_error) if the device cannot be queried.  Launches nothing.
 */
int pa_device_memory(int device, int* bus_width_bits, int* mem_clock_khz);

/*
 * pa_check_inputs_host -- validate HOST copies of the device data against the
 * contract above: 0 <= L <= max_blocks_per_seq * block_size, every table entry
 * in use in [0, num_blocks), and, if check_write_targets is nonzero, that no
 * two sequences' newest tokens map to the same (block, row).  Returns PA_OK or
 * PA_ERR_INVALID_ARG; on failure *bad_seq (if not NULL) receives the first
 * offending sequence and pa_last_error() says what is wrong.  Pure host code.
 */
int pa_check_inputs_host(const int32_t* block_tables, const int32_t* context_lens,
                         int num_seqs, int block_size, int max_blocks_per_seq,
                         int num_blocks, int check_write_targets, int* bad_seq);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
