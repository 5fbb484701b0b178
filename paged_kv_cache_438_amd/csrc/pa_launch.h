// Internal interface between the C ABI (pa_api.cpp) and the HIP kernels
// (pa_kernels.hip).  Not installed; callers use include/pa.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace pa {

enum Dtype : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// Decode flag bits (PA_FLAG_* in pa.h).
constexpr int kFlagSharedKV = 1;
constexpr int kFlagValuOnly = 2;

struct CacheWriteParams;

struct DecodeParams {
  void* out;
  const void* q;
  const void* k_pool;
  const void* v_pool;
  const int32_t* block_tables;  // nullptr: a contiguous cache of max_len rows per sequence
  const int32_t* context_lens;
  float* workspace;        // split-K partials; nullptr for a single pass
  int num_seqs;
  int num_heads;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int max_blocks_per_seq;
  int num_blocks;
  float scale;
  int dtype;
  int partition_size;      // tokens per partition (multiple of 16)
  int max_partitions;      // partitions per sequence covered by the grid
  int flags;               // PA_FLAG_* bits
  int max_len;             // contiguous cache: rows per (sequence, KV head); 0 when paged
  // Shared-prompt decode (seq_group == nullptr otherwise).
  const int32_t* seq_group;     // [num_seqs] group of each sequence or -1
  const int32_t* group_prefix;  // [num_groups] shared prompt tokens of each group
  int num_groups;
  int max_group_size;
  // The new token's write done in the same call (nullptr: none); with a
  // split-K workspace it runs in the plan's launch.
  const CacheWriteParams* write;
};

struct CacheWriteParams {
  void* k_pool;
  void* v_pool;
  const void* k_new;
  const void* v_new;
  const int32_t* block_tables;  // nullptr: a contiguous cache of max_len rows per sequence
  const int32_t* context_lens;
  int num_seqs;
  int num_kv_heads;
  int head_dim;
  int block_size;
  int max_blocks_per_seq;
  int num_blocks;
  int dtype;
  int max_len;             // contiguous cache: rows per (sequence, KV head); 0 when paged
};

// Byte offsets of the parts of the split-K workspace (pa_workspace.cpp).
struct WsLayout {
  size_t max_units;   // capacity of the unit list
  size_t ml, n_units, units, split, minfo, arrival, group_fill, group_start, group_lp, total;
};
// Bytes of one unit record of the plan.
constexpr size_t kUnitRecordBytes = 32;
WsLayout ws_layout(int num_seqs, int num_heads, int head_dim, int max_partitions,
                   int num_groups);
// Byte size of the split-K workspace for these sizes: partials and plan;
// num_groups >= 0 (shared-prompt decode) adds the group tables, -1 does not.
size_t splitk_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_partitions,
                              int num_groups);

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream);
// Block moves between a device pool and a host pool's device mapping; pairs
// is a host array, already checked against both pools.
hipError_t launch_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* pairs, int num_pairs, size_t block_bytes,
                              hipStream_t stream);
hipError_t launch_read_probe(const void* buf, size_t tile_bytes, const int32_t* order,
                             int ntiles, uint32_t* sink, hipStream_t stream);
hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int num_pairs,
                              int num_blocks, size_t block_bytes, hipStream_t stream);
// Single pass when p.workspace == nullptr (then p.max_partitions must be 1).
hipError_t launch_decode(const DecodeParams& p, hipStream_t stream);

// Size of the library's static device scratch (PA_NOALLOC_SCRATCH_BYTES in
// pa.h), which holds the split-K workspace for callers that cannot allocate.
constexpr size_t kNoallocScratchBytes = (size_t)32 << 20;
// Device address of that scratch on the current device.  The address is
// looked up once per device (hipGetSymbolAddress, with the device current)
// and kept; nothing is allocated.
hipError_t noalloc_scratch(void** ptr);

}  // namespace pa
