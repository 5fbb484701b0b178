// C ABI of libpa (declared in include/pa.h): host-side argument checks,
// then one or two kernel launches on the caller's stream.  No allocation,
// no synchronisation, no device-to-host copy.
#include "pa.h"

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <string>
#include <unordered_set>

#include "pa_errors.h"
#include "pa_launch.h"

namespace {
thread_local std::string g_last_error;
}  // namespace

int pa_fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

int pa_ok() {
  g_last_error.clear();
  return PA_OK;
}

namespace {

bool is_pow2(int x) { return x > 0 && (x & (x - 1)) == 0; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_common(int num_seqs, int num_kv_heads, int head_dim, int block_size,
                 int max_blocks_per_seq, int num_blocks, int dtype) {
  if (num_seqs < 0) return pa_fail(PA_ERR_INVALID_ARG, "num_seqs must be >= 0 (got %d)", num_seqs);
  if (num_kv_heads <= 0) return pa_fail(PA_ERR_INVALID_ARG, "num_kv_heads must be > 0 (got %d)", num_kv_heads);
  if (max_blocks_per_seq <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq must be > 0 (got %d)", max_blocks_per_seq);
  if (num_blocks <= 0) return pa_fail(PA_ERR_INVALID_ARG, "num_blocks must be > 0 (got %d)", num_blocks);
  if (head_dim != 64 && head_dim != 128)
    return pa_fail(PA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (!is_pow2(block_size) || block_size > 65536)
    return pa_fail(PA_ERR_UNSUPPORTED, "block_size %d not supported (power of two in [1,65536])",
                   block_size);
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16)
    return pa_fail(PA_ERR_UNSUPPORTED, "unknown dtype %d", dtype);
  if ((long long)max_blocks_per_seq * block_size > 0x3fffffffLL)
    return pa_fail(PA_ERR_INVALID_ARG, "max_blocks_per_seq * block_size too large");
  return PA_OK;
}

int check_decode(const void* out, const void* q, const void* k_pool, const void* v_pool,
                 const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                 int num_heads, int num_kv_heads, int head_dim, int block_size,
                 int max_blocks_per_seq, int num_blocks, float scale, int dtype, int flags) {
  int st = check_common(num_seqs, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, dtype);
  if (st) return st;
  if (num_heads <= 0) return pa_fail(PA_ERR_INVALID_ARG, "num_heads must be > 0 (got %d)", num_heads);
  if (num_heads % num_kv_heads != 0)
    return pa_fail(PA_ERR_INVALID_ARG, "num_heads %d is not a multiple of num_kv_heads %d", num_heads,
                num_kv_heads);
  if (flags & ~(PA_FLAG_SHARED_KV | PA_FLAG_VALU_ONLY)) return pa_fail(PA_ERR_INVALID_ARG, "unknown flag bits 0x%x", flags);
  if (!(scale == scale) || scale == __builtin_inff() || scale == -__builtin_inff())
    return pa_fail(PA_ERR_INVALID_ARG, "scale must be finite");
  if (num_seqs == 0) return PA_OK;
  if (!out || !q || !k_pool || !v_pool || !block_tables || !context_lens)
    return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(q) || !aligned16(k_pool) || !aligned16(v_pool))
    return pa_fail(PA_ERR_INVALID_ARG, "q, k_pool and v_pool must be 16-byte aligned");
  if (!aligned16(out))
    return pa_fail(PA_ERR_INVALID_ARG, "out must be 16-byte aligned");
  return PA_OK;
}

pa::DecodeParams make_params(void* out, const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int num_blocks,
                             float scale, int dtype, int flags) {
  pa::DecodeParams p;
  p.out = out;
  p.q = q;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.workspace = nullptr;
  p.num_seqs = num_seqs;
  p.num_heads = num_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.scale = scale;
  p.dtype = dtype;
  p.partition_size = 0;
  p.max_partitions = 1;
  p.flags = flags;
  p.max_len = 0;
  p.seq_group = nullptr;
  p.group_prefix = nullptr;
  p.num_groups = 0;
  p.max_group_size = 1;
  p.write = nullptr;
  return p;
}

int finish_launch(hipError_t e) {
  if (e != hipSuccess) return pa_fail(PA_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return pa_ok();
}

int64_t ceil_div64(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

extern "C" {

int pa_abi_version(void) { return PA_ABI_VERSION; }

const char* pa_status_str(int status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_NULL: return "null pointer";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP runtime error";
    case PA_ERR_OUT_OF_BLOCKS: return "too few free blocks";
    default: return "unknown status";
  }
}

const char* pa_last_error(void) { return g_last_error.c_str(); }

int pa_cache_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                   const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                   int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                   int num_blocks, int dtype, void* stream) {
  int st = check_common(num_seqs, num_kv_heads, head_dim, block_size, max_blocks_per_seq,
                        num_blocks, dtype);
  if (st) return st;
  if (num_seqs == 0) return pa_ok();
  if (!k_pool || !v_pool || !k_new || !v_new || !block_tables || !context_lens)
    return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(k_pool) || !aligned16(v_pool) || !aligned16(k_new) || !aligned16(v_new))
    return pa_fail(PA_ERR_INVALID_ARG, "pools and new rows must be 16-byte aligned");
  pa::CacheWriteParams p;
  p.k_pool = k_pool;
  p.v_pool = v_pool;
  p.k_new = k_new;
  p.v_new = v_new;
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.num_blocks = num_blocks;
  p.dtype = dtype;
  p.max_len = 0;
  return finish_launch(pa::launch_cache_write(p, static_cast<hipStream_t>(stream)));
}

int pa_cache_write_contiguous(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                              const int32_t* context_lens, int num_seqs, int num_kv_heads,
                              int head_dim, int max_len, int dtype, void* stream) {
  if (max_len <= 0) return pa_fail(PA_ERR_INVALID_ARG, "max_len must be > 0 (got %d)", max_len);
  // The checks of a paged call with one block of max_len rows per sequence.
  int st = check_common(num_seqs, num_kv_heads, head_dim, 1, max_len, num_seqs > 0 ? num_seqs : 1,
                        dtype);
  if (st) return st;
  if (num_seqs == 0) return pa_ok();
  if (!k_cache || !v_cache || !k_new || !v_new || !context_lens)
    return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_new) || !aligned16(v_new))
    return pa_fail(PA_ERR_INVALID_ARG, "caches and new rows must be 16-byte aligned");
  pa::CacheWriteParams p;
  p.k_pool = k_cache;
  p.v_pool = v_cache;
  p.k_new = k_new;
  p.v_new = v_new;
  p.block_tables = nullptr;
  p.context_lens = context_lens;
  p.num_seqs = num_seqs;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = 1;
  p.max_blocks_per_seq = 1;
  p.num_blocks = num_seqs;
  p.dtype = dtype;
  p.max_len = max_len;
  return finish_launch(pa::launch_cache_write(p, static_cast<hipStream_t>(stream)));
}

int pa_decode(void* out, const void* q, const void* k_pool, const void* v_pool,
              const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
              int num_heads, int num_kv_heads, int head_dim, int block_size,
              int max_blocks_per_seq, int num_blocks, float scale, int dtype, int flags,
              void* stream) {
  int st = check_decode(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                        num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                        dtype, flags);
  if (st) return st;
  if (num_seqs == 0) return pa_ok();
  pa::DecodeParams p = make_params(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs,
                                   num_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, num_blocks, scale, dtype, flags);
  // One partition spanning the longest sequence the tables can describe.
  p.partition_size = (int)(ceil_div64((int64_t)max_blocks_per_seq * block_size, 16) * 16);
  p.max_partitions = 1;
  return finish_launch(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

size_t pa_decode_splitk_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                        int max_context_len, int partition_size) {
  if (num_seqs < 0 || num_heads <= 0 || (head_dim != 64 && head_dim != 128) ||
      max_context_len < 0 || partition_size <= 0 || partition_size % 16 != 0)
    return 0;
  const int parts = (int)ceil_div64(max_context_len, partition_size);
  const size_t bytes =
      pa::splitk_workspace_bytes(num_seqs, num_heads, head_dim, parts > 0 ? parts : 1, -1);
  return (bytes + 255) / 256 * 256;
}

// A shared prompt can split one partition of a sequence in two (prompt tail
// and own head), hence one partition more than the plain split.
static int shared_parts(int max_context_len, int partition_size) {
  return (int)ceil_div64(max_context_len, partition_size) + 1;
}

size_t pa_decode_shared_prefix_workspace_bytes(int num_seqs, int num_heads, int head_dim,
                                               int max_context_len, int partition_size,
                                               int num_groups) {
  if (num_seqs < 0 || num_heads <= 0 || (head_dim != 64 && head_dim != 128) ||
      max_context_len < 0 || partition_size <= 0 || partition_size % 16 != 0 || num_groups < 0)
    return 0;
  const size_t bytes = pa::splitk_workspace_bytes(
      num_seqs, num_heads, head_dim, shared_parts(max_context_len, partition_size), num_groups);
  return (bytes + 255) / 256 * 256;
}

}  // extern "C"

namespace {

int shared_prefix_impl(void* out, const void* q, const void* k_pool, const void* v_pool,
                       const int32_t* block_tables, const int32_t* context_lens,
                       const int32_t* seq_group, const int32_t* group_prefix_len, int num_seqs,
                       int num_heads, int num_kv_heads, int head_dim, int block_size,
                       int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                       int num_groups, int max_group_size, int partition_size,
                       int max_context_len, void* workspace, size_t workspace_bytes, int flags,
                       const pa::CacheWriteParams* write, void* stream) {
  int st = check_decode(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                        num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                        dtype, flags);
  if (st) return st;
  if (dtype != PA_F16 && dtype != PA_BF16)
    return pa_fail(PA_ERR_UNSUPPORTED, "shared-prefix decode runs on the matrix cores: fp16 or bf16");
  if (flags & PA_FLAG_VALU_ONLY)
    return pa_fail(PA_ERR_INVALID_ARG, "PA_FLAG_VALU_ONLY does not apply to shared-prefix decode");
  if (partition_size <= 0 || partition_size % 16 != 0)
    return pa_fail(PA_ERR_INVALID_ARG, "partition_size must be a positive multiple of 16 (got %d)",
                partition_size);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return pa_fail(PA_ERR_INVALID_ARG,
                "max_context_len %d outside [0, max_blocks_per_seq*block_size = %lld]",
                max_context_len, (long long)max_blocks_per_seq * block_size);
  if (num_groups < 0) return pa_fail(PA_ERR_INVALID_ARG, "num_groups must be >= 0 (got %d)", num_groups);
  if (max_group_size < 1 || max_group_size > num_seqs + (num_seqs == 0))
    return pa_fail(PA_ERR_INVALID_ARG, "max_group_size %d outside [1, num_seqs]", max_group_size);
  if ((int64_t)max_group_size * (num_heads / num_kv_heads) > 4096)
    return pa_fail(PA_ERR_INVALID_ARG, "max_group_size * query heads per KV head exceeds 4096");
  if (num_seqs == 0) return pa_ok();
  if (!seq_group || (num_groups > 0 && !group_prefix_len))
    return pa_fail(PA_ERR_NULL, "seq_group and group_prefix_len are required");
  const size_t need = pa_decode_shared_prefix_workspace_bytes(
      num_seqs, num_heads, head_dim, max_context_len, partition_size, num_groups);
  if (!workspace || workspace_bytes < need)
    return pa_fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return pa_fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  pa::DecodeParams p = make_params(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs,
                                   num_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, num_blocks, scale, dtype, flags);
  p.partition_size = partition_size;
  p.max_partitions = shared_parts(max_context_len, partition_size);
  p.workspace = static_cast<float*>(workspace);
  p.seq_group = seq_group;
  p.group_prefix = group_prefix_len;
  p.num_groups = num_groups;
  p.max_group_size = max_group_size;
  p.write = write;
  return finish_launch(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

// The new-token write of a combined call: the paged pools and tables of the
// decode.  Checked here only for what the decode's checks do not cover.
int new_rows_check(int num_seqs, const void* k_new, const void* v_new) {
  if (num_seqs == 0) return PA_OK;
  if (!k_new || !v_new) return pa_fail(PA_ERR_NULL, "k_new and v_new are required");
  if (!aligned16(k_new) || !aligned16(v_new))
    return pa_fail(PA_ERR_INVALID_ARG, "k_new and v_new must be 16-byte aligned");
  return PA_OK;
}

pa::CacheWriteParams make_write(void* k_pool, void* v_pool, const void* k_new, const void* v_new,
                                const int32_t* block_tables, const int32_t* context_lens,
                                int num_seqs, int num_kv_heads, int head_dim, int block_size,
                                int max_blocks_per_seq, int num_blocks, int dtype) {
  pa::CacheWriteParams w;
  w.k_pool = k_pool;
  w.v_pool = v_pool;
  w.k_new = k_new;
  w.v_new = v_new;
  w.block_tables = block_tables;
  w.context_lens = context_lens;
  w.num_seqs = num_seqs;
  w.num_kv_heads = num_kv_heads;
  w.head_dim = head_dim;
  w.block_size = block_size;
  w.max_blocks_per_seq = max_blocks_per_seq;
  w.num_blocks = num_blocks;
  w.dtype = dtype;
  w.max_len = 0;
  return w;
}

}  // namespace

extern "C" {

int pa_decode_shared_prefix(void* out, const void* q, const void* k_pool, const void* v_pool,
                            const int32_t* block_tables, const int32_t* context_lens,
                            const int32_t* seq_group, const int32_t* group_prefix_len,
                            int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                            int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                            int dtype, int num_groups, int max_group_size, int partition_size,
                            int max_context_len, void* workspace, size_t workspace_bytes,
                            int flags, void* stream) {
  return shared_prefix_impl(out, q, k_pool, v_pool, block_tables, context_lens, seq_group,
                            group_prefix_len, num_seqs, num_heads, num_kv_heads, head_dim,
                            block_size, max_blocks_per_seq, num_blocks, scale, dtype, num_groups,
                            max_group_size, partition_size, max_context_len, workspace,
                            workspace_bytes, flags, nullptr, stream);
}

int pa_write_decode(void* out, const void* q, void* k_pool, void* v_pool, const void* k_new,
                    const void* v_new, const int32_t* block_tables, const int32_t* context_lens,
                    int num_seqs, int num_heads, int num_kv_heads, int head_dim, int block_size,
                    int max_blocks_per_seq, int num_blocks, float scale, int dtype, int flags,
                    void* stream) {
  int st = check_decode(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                        num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                        dtype, flags);
  if (st) return st;
  st = new_rows_check(num_seqs, k_new, v_new);
  if (st) return st;
  if (num_seqs == 0) return pa_ok();
  pa::DecodeParams p = make_params(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs,
                                   num_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, num_blocks, scale, dtype, flags);
  p.partition_size = (int)(ceil_div64((int64_t)max_blocks_per_seq * block_size, 16) * 16);
  p.max_partitions = 1;
  const pa::CacheWriteParams w =
      make_write(k_pool, v_pool, k_new, v_new, block_tables, context_lens, num_seqs,
                 num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, dtype);
  p.write = &w;
  return finish_launch(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int pa_write_decode_shared_prefix(void* out, const void* q, void* k_pool, void* v_pool,
                                  const void* k_new, const void* v_new,
                                  const int32_t* block_tables, const int32_t* context_lens,
                                  const int32_t* seq_group, const int32_t* group_prefix_len,
                                  int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                                  int block_size, int max_blocks_per_seq, int num_blocks,
                                  float scale, int dtype, int num_groups, int max_group_size,
                                  int partition_size, int max_context_len, void* workspace,
                                  size_t workspace_bytes, int flags, void* stream) {
  const int st = new_rows_check(num_seqs, k_new, v_new);
  if (st) return st;
  const pa::CacheWriteParams w =
      make_write(k_pool, v_pool, k_new, v_new, block_tables, context_lens, num_seqs,
                 num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, dtype);
  return shared_prefix_impl(out, q, k_pool, v_pool, block_tables, context_lens, seq_group,
                            group_prefix_len, num_seqs, num_heads, num_kv_heads, head_dim,
                            block_size, max_blocks_per_seq, num_blocks, scale, dtype, num_groups,
                            max_group_size, partition_size, max_context_len, workspace,
                            workspace_bytes, flags, &w, stream);
}

}  // extern "C"

namespace {

// Checks and launch shared by the two split-K entries; `workspace` is the
// caller's buffer or the library's static scratch.
int splitk_checks(void* out, const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                  int num_heads, int num_kv_heads, int head_dim, int block_size,
                  int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                  int partition_size, int max_context_len, int flags) {
  int st = check_decode(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                        num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                        dtype, flags);
  if (st) return st;
  if (partition_size <= 0 || partition_size % 16 != 0)
    return pa_fail(PA_ERR_INVALID_ARG, "partition_size must be a positive multiple of 16 (got %d)",
                partition_size);
  if (max_context_len < 0 || (int64_t)max_context_len > (int64_t)max_blocks_per_seq * block_size)
    return pa_fail(PA_ERR_INVALID_ARG,
                "max_context_len %d outside [0, max_blocks_per_seq*block_size = %lld]",
                max_context_len, (long long)max_blocks_per_seq * block_size);
  return PA_OK;
}

int splitk_launch(void* out, const void* q, const void* k_pool, const void* v_pool,
                  const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                  int num_heads, int num_kv_heads, int head_dim, int block_size,
                  int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                  int partition_size, int max_context_len, void* workspace, int flags,
                  void* stream, const pa::CacheWriteParams* write = nullptr) {
  pa::DecodeParams p = make_params(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs,
                                   num_heads, num_kv_heads, head_dim, block_size,
                                   max_blocks_per_seq, num_blocks, scale, dtype, flags);
  const int parts = (int)ceil_div64(max_context_len, partition_size);
  p.partition_size = partition_size;
  p.max_partitions = parts > 0 ? parts : 1;
  p.workspace = static_cast<float*>(workspace);
  p.write = write;
  return finish_launch(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

int pa_decode_splitk(void* out, const void* q, const void* k_pool, const void* v_pool,
                     const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                     int num_heads, int num_kv_heads, int head_dim, int block_size,
                     int max_blocks_per_seq, int num_blocks, float scale, int dtype,
                     int partition_size, int max_context_len, void* workspace,
                     size_t workspace_bytes, int flags, void* stream) {
  int st = splitk_checks(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                         num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                         scale, dtype, partition_size, max_context_len, flags);
  if (st) return st;
  if (num_seqs == 0) return pa_ok();
  const size_t need = pa_decode_splitk_workspace_bytes(num_seqs, num_heads, head_dim,
                                                       max_context_len, partition_size);
  if (!workspace || workspace_bytes < need)
    return pa_fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return pa_fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  return splitk_launch(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       dtype, partition_size, max_context_len, workspace, flags, stream);
}

int pa_write_decode_splitk(void* out, const void* q, void* k_pool, void* v_pool,
                           const void* k_new, const void* v_new, const int32_t* block_tables,
                           const int32_t* context_lens, int num_seqs, int num_heads,
                           int num_kv_heads, int head_dim, int block_size, int max_blocks_per_seq,
                           int num_blocks, float scale, int dtype, int partition_size,
                           int max_context_len, void* workspace, size_t workspace_bytes,
                           int flags, void* stream) {
  int st = splitk_checks(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                         num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                         scale, dtype, partition_size, max_context_len, flags);
  if (st) return st;
  st = new_rows_check(num_seqs, k_new, v_new);
  if (st) return st;
  if (num_seqs == 0) return pa_ok();
  const size_t need = pa_decode_splitk_workspace_bytes(num_seqs, num_heads, head_dim,
                                                       max_context_len, partition_size);
  if (!workspace || workspace_bytes < need)
    return pa_fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need,
                workspace_bytes, workspace ? "" : ", NULL");
  if (!aligned16(workspace)) return pa_fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
  const pa::CacheWriteParams w =
      make_write(k_pool, v_pool, k_new, v_new, block_tables, context_lens, num_seqs,
                 num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, dtype);
  return splitk_launch(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       dtype, partition_size, max_context_len, workspace, flags, stream, &w);
}

int pa_decode_splitk_noalloc(void* out, const void* q, const void* k_pool, const void* v_pool,
                             const int32_t* block_tables, const int32_t* context_lens,
                             int num_seqs, int num_heads, int num_kv_heads, int head_dim,
                             int block_size, int max_blocks_per_seq, int num_blocks, float scale,
                             int dtype, int partition_size, int max_context_len, int flags,
                             void* stream) {
  static_assert(PA_NOALLOC_SCRATCH_BYTES == pa::kNoallocScratchBytes, "scratch size");
  int st = splitk_checks(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                         num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks,
                         scale, dtype, partition_size, max_context_len, flags);
  if (st) return st;
  if (num_seqs == 0) return pa_ok();
  const size_t need = pa_decode_splitk_workspace_bytes(num_seqs, num_heads, head_dim,
                                                       max_context_len, partition_size);
  if (need > PA_NOALLOC_SCRATCH_BYTES)
    return pa_fail(PA_ERR_WORKSPACE,
                   "these sizes need %zu bytes of split-K workspace but the static scratch holds "
                   "%zu; use pa_decode_splitk with a caller workspace, a larger partition_size "
                   "or fewer sequences", need, (size_t)PA_NOALLOC_SCRATCH_BYTES);
  void* ws = nullptr;
  const hipError_t e = pa::noalloc_scratch(&ws);
  if (e != hipSuccess)
    return pa_fail(PA_ERR_HIP, "static scratch address: %s", hipGetErrorString(e));
  return splitk_launch(out, q, k_pool, v_pool, block_tables, context_lens, num_seqs, num_heads,
                       num_kv_heads, head_dim, block_size, max_blocks_per_seq, num_blocks, scale,
                       dtype, partition_size, max_context_len, ws, flags, stream);
}

int pa_decode_contiguous(void* out, const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* context_lens, int num_seqs, int num_heads,
                         int num_kv_heads, int head_dim, int max_len, float scale, int dtype,
                         int partition_size, void* workspace, size_t workspace_bytes, int flags,
                         void* stream) {
  if (max_len <= 0) return pa_fail(PA_ERR_INVALID_ARG, "max_len must be > 0 (got %d)", max_len);
  if (flags & PA_FLAG_SHARED_KV)
    return pa_fail(PA_ERR_INVALID_ARG, "PA_FLAG_SHARED_KV does not apply to a contiguous cache");
  // The checks of a paged call whose one block per sequence holds max_len
  // rows (block_size 1 stands in for the size, which need not be a power of
  // two); the table pointer is not used.
  int st = check_decode(out, q, k_cache, v_cache, context_lens, context_lens, num_seqs,
                        num_heads, num_kv_heads, head_dim, 1, max_len, num_seqs > 0 ? num_seqs : 1,
                        scale, dtype, flags);
  if (st) return st;
  if ((int64_t)max_len * head_dim * (dtype == PA_F32 ? 4 : 2) > 0x7fffffffLL)
    return pa_fail(PA_ERR_UNSUPPORTED, "max_len %d: one sequence's rows of a KV head exceed 2 GiB",
                   max_len);
  if (partition_size < 0 || partition_size % 16 != 0)
    return pa_fail(PA_ERR_INVALID_ARG,
                   "partition_size must be 0 (single pass) or a positive multiple of 16 (got %d)",
                   partition_size);
  if (num_seqs == 0) return pa_ok();
  pa::DecodeParams p = make_params(out, q, k_cache, v_cache, nullptr, context_lens, num_seqs,
                                   num_heads, num_kv_heads, head_dim, 1, 1, num_seqs, scale,
                                   dtype, flags);
  p.max_len = max_len;
  if (partition_size == 0) {
    p.partition_size = (int)(ceil_div64(max_len, 16) * 16);
    p.max_partitions = 1;
  } else {
    const size_t need = pa_decode_splitk_workspace_bytes(num_seqs, num_heads, head_dim, max_len,
                                                         partition_size);
    if (!workspace || workspace_bytes < need)
      return pa_fail(PA_ERR_WORKSPACE, "workspace of %zu bytes needed (got %zu%s)", need,
                     workspace_bytes, workspace ? "" : ", NULL");
    if (!aligned16(workspace))
      return pa_fail(PA_ERR_INVALID_ARG, "workspace must be 16-byte aligned");
    p.partition_size = partition_size;
    p.max_partitions = (int)ceil_div64(max_len, partition_size);
    p.workspace = static_cast<float*>(workspace);
  }
  return finish_launch(pa::launch_decode(p, static_cast<hipStream_t>(stream)));
}

int pa_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int num_pairs,
                   int num_kv_heads, int head_dim, int block_size, int num_blocks, int dtype,
                   void* stream) {
  int st = check_common(1, num_kv_heads, head_dim, block_size, 1, num_blocks, dtype);
  if (st) return st;
  if (num_pairs < 0) return pa_fail(PA_ERR_INVALID_ARG, "num_pairs must be >= 0 (got %d)", num_pairs);
  if (num_pairs > 65535) return pa_fail(PA_ERR_INVALID_ARG, "at most 65535 pairs per call");
  if (num_pairs == 0) return pa_ok();
  if (!k_pool || !v_pool || !pairs) return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(k_pool) || !aligned16(v_pool))
    return pa_fail(PA_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  const size_t block_bytes = (size_t)num_kv_heads * block_size * head_dim * (dtype == PA_F32 ? 4 : 2);
  return finish_launch(pa::launch_copy_blocks(k_pool, v_pool, pairs, num_pairs, num_blocks,
                                              block_bytes, static_cast<hipStream_t>(stream)));
}

int pa_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                   const int32_t* pairs, int num_pairs, int num_dst_blocks, int num_src_blocks,
                   size_t block_bytes, int to_host, void* stream) {
  if (num_pairs < 0 || num_dst_blocks < 0 || num_src_blocks < 0 || block_bytes == 0)
    return pa_fail(PA_ERR_INVALID_ARG, "invalid sizes");
  if (num_pairs == 0) return pa_ok();
  if (!dst_k || !dst_v || !src_k || !src_v || !pairs)
    return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  for (int i = 0; i < num_pairs; ++i)
    if (pairs[2 * i] < 0 || pairs[2 * i] >= num_src_blocks || pairs[2 * i + 1] < 0 ||
        pairs[2 * i + 1] >= num_dst_blocks)
      return pa_fail(PA_ERR_INVALID_ARG, "pair %d (%d, %d) outside the pools", i, pairs[2 * i],
                     pairs[2 * i + 1]);
  const hipMemcpyKind kind = to_host ? hipMemcpyDeviceToHost : hipMemcpyHostToDevice;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (block_bytes % 16 == 0) {
    // Many short runs: one kernel moves every block through the host pool's
    // device mapping, when the host pool is pinned memory that has one.
    int runs = 1;
    for (int i = 1; i < num_pairs; ++i)
      runs += !(pairs[2 * i] == pairs[2 * (i - 1)] + 1 &&
                pairs[2 * i + 1] == pairs[2 * (i - 1) + 1] + 1);
    if (runs > 8 && (size_t)num_pairs * block_bytes / runs < ((size_t)4 << 20)) {
      void* host_k = to_host ? dst_k : const_cast<void*>(src_k);
      void* host_v = to_host ? dst_v : const_cast<void*>(src_v);
      void* mk = nullptr;
      void* mv = nullptr;
      // An error left by an earlier call is the caller's: clear only the one
      // a failed lookup below leaves.
      const bool clean_before = hipPeekAtLastError() == hipSuccess;
      if (hipHostGetDevicePointer(&mk, host_k, 0) == hipSuccess &&
          hipHostGetDevicePointer(&mv, host_v, 0) == hipSuccess && mk && mv) {
        const hipError_t e =
            to_host ? pa::launch_swap_blocks(mk, mv, src_k, src_v, pairs, num_pairs, block_bytes, st)
                    : pa::launch_swap_blocks(dst_k, dst_v, mk, mv, pairs, num_pairs, block_bytes, st);
        if (e != hipSuccess) return pa_fail(PA_ERR_HIP, "swap launch failed: %s", hipGetErrorString(e));
        return pa_ok();
      }
      if (clean_before) (void)hipGetLastError();   // not mapped: copy below
    }
  }
  // Runs of pairs whose sources and destinations are both consecutive go out
  // as one copy per pool.
  for (int i = 0; i < num_pairs;) {
    int j = i + 1;
    while (j < num_pairs && pairs[2 * j] == pairs[2 * (j - 1)] + 1 &&
           pairs[2 * j + 1] == pairs[2 * (j - 1) + 1] + 1)
      ++j;
    const size_t bytes = (size_t)(j - i) * block_bytes;
    const size_t so = (size_t)pairs[2 * i] * block_bytes, dso = (size_t)pairs[2 * i + 1] * block_bytes;
    hipError_t e = hipMemcpyAsync(static_cast<uint8_t*>(dst_k) + dso,
                                  static_cast<const uint8_t*>(src_k) + so, bytes, kind, st);
    if (e == hipSuccess)
      e = hipMemcpyAsync(static_cast<uint8_t*>(dst_v) + dso, static_cast<const uint8_t*>(src_v) + so,
                         bytes, kind, st);
    if (e != hipSuccess) return pa_fail(PA_ERR_HIP, "copy failed: %s", hipGetErrorString(e));
    i = j;
  }
  return pa_ok();
}

int pa_read_probe(const void* buf, size_t tile_bytes, const int32_t* tile_order, int num_tiles,
                  uint32_t* sink, void* stream) {
  if (num_tiles < 0 || tile_bytes == 0 || tile_bytes % 4096 != 0)
    return pa_fail(PA_ERR_INVALID_ARG, "tile_bytes must be a positive multiple of 4096 and "
                                       "num_tiles >= 0");
  if (num_tiles == 0) return pa_ok();
  if (!buf || !tile_order || !sink) return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  if (!aligned16(buf)) return pa_fail(PA_ERR_INVALID_ARG, "buf must be 16-byte aligned");
  return finish_launch(pa::launch_read_probe(buf, tile_bytes, tile_order, num_tiles, sink,
                                             static_cast<hipStream_t>(stream)));
}

int pa_device_memory(int device, int* bus_width_bits, int* mem_clock_khz) {
  if (!bus_width_bits || !mem_clock_khz) return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  hipError_t e = hipDeviceGetAttribute(bus_width_bits, hipDeviceAttributeMemoryBusWidth, device);
  if (e == hipSuccess)
    e = hipDeviceGetAttribute(mem_clock_khz, hipDeviceAttributeMemoryClockRate, device);
  if (e != hipSuccess) return pa_fail(PA_ERR_HIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
  return pa_ok();
}

int pa_check_inputs_host(const int32_t* block_tables, const int32_t* context_lens, int num_seqs,
                         int block_size, int max_blocks_per_seq, int num_blocks,
                         int check_write_targets, int* bad_seq) {
  if (bad_seq) *bad_seq = -1;
  if (num_seqs < 0 || block_size <= 0 || max_blocks_per_seq <= 0 || num_blocks <= 0)
    return pa_fail(PA_ERR_INVALID_ARG, "invalid sizes");
  if (num_seqs == 0) return pa_ok();
  if (!block_tables || !context_lens) return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  const int64_t cap = (int64_t)max_blocks_per_seq * block_size;
  std::unordered_set<int64_t> slots;
  for (int s = 0; s < num_seqs; ++s) {
    const int64_t L = context_lens[s];
    if (L < 0 || L > cap) {
      if (bad_seq) *bad_seq = s;
      return pa_fail(PA_ERR_INVALID_ARG, "sequence %d: length %lld outside [0, %lld]", s,
                  (long long)L, (long long)cap);
    }
    const int64_t nb = ceil_div64(L, block_size);
    const int32_t* row = block_tables + (size_t)s * max_blocks_per_seq;
    for (int64_t i = 0; i < nb; ++i) {
      if (row[i] < 0 || row[i] >= num_blocks) {
        if (bad_seq) *bad_seq = s;
        return pa_fail(PA_ERR_INVALID_ARG, "sequence %d: block table entry %lld = %d outside [0, %d)",
                    s, (long long)i, row[i], num_blocks);
      }
    }
    if (check_write_targets && L >= 1) {
      const int64_t pos = L - 1;
      const int64_t slot = (int64_t)row[pos / block_size] * block_size + pos % block_size;
      if (!slots.insert(slot).second) {
        if (bad_seq) *bad_seq = s;
        return pa_fail(PA_ERR_INVALID_ARG,
                    "sequence %d: new-token slot (block %d, row %lld) already written by another "
                    "sequence", s, row[pos / block_size], (long long)(pos % block_size));
      }
    }
  }
  return pa_ok();
}

}  // extern "C"
