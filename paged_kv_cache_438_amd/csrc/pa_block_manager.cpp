// Host-side block manager (include/pa_block_manager.h): free lists, reference
// counts, copy-on-write and swap bookkeeping for the paged KV cache.  Plain
// C++; it never touches the GPU.
#include "pa_block_manager.h"

#include <algorithm>
#include <set>
#include <string>
#include <unordered_map>
#include <vector>

#include "pa_errors.h"

struct pa_bm {
  struct Seq {
    int dev;                 // 0 GPU, 1 CPU
    std::vector<int> ids;    // blocks in logical order
    int64_t tokens;
  };
  int bs = 0;
  std::vector<int> ref[2];   // reference count per block
  std::set<int> free_[2];    // free blocks, lowest id first
  std::unordered_map<int, Seq> seqs;

  int64_t blocks_needed(int64_t tokens) const { return (tokens + bs - 1) / bs; }

  // n free blocks of device dev (lowest first), each with count 1; the
  // caller has checked that enough are free.
  std::vector<int> take(int dev, int64_t n) {
    std::vector<int> out;
    out.reserve((size_t)n);
    auto it = free_[dev].begin();
    for (int64_t i = 0; i < n; ++i) {
      const int b = *it;
      it = free_[dev].erase(it);
      ref[dev][b] = 1;
      out.push_back(b);
    }
    return out;
  }
  void release(int dev, int b) {
    if (--ref[dev][b] == 0) free_[dev].insert(b);
  }
};

namespace {

pa_bm::Seq* find(pa_bm* bm, int seq_id) {
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? nullptr : &it->second;
}
const pa_bm::Seq* find(const pa_bm* bm, int seq_id) {
  auto it = bm->seqs.find(seq_id);
  return it == bm->seqs.end() ? nullptr : &it->second;
}

int swap(pa_bm* bm, int seq_id, int from, int32_t* pairs, int max_pairs, int* num_pairs) {
  if (!bm) return pa_fail(PA_ERR_NULL, "manager is NULL");
  pa_bm::Seq* s = find(bm, seq_id);
  if (!s) return pa_fail(PA_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  if (s->dev != from)
    return pa_fail(PA_ERR_INVALID_ARG, "sequence %d is not on the %s", seq_id, from ? "CPU" : "GPU");
  for (int b : s->ids)
    if (bm->ref[from][b] > 1)
      return pa_fail(PA_ERR_INVALID_ARG, "sequence %d shares block %d; swap refused", seq_id, b);
  const int to = 1 - from;
  const int64_t n = (int64_t)s->ids.size();
  if (n > max_pairs || (n > 0 && !pairs))
    return pa_fail(PA_ERR_INVALID_ARG, "%lld block pairs need room (max_pairs %d)", (long long)n,
                   max_pairs);
  if ((int64_t)bm->free_[to].size() < n)
    return pa_fail(PA_ERR_OUT_OF_BLOCKS, "%lld free %s blocks needed, %zu free", (long long)n,
                   to ? "CPU" : "GPU", bm->free_[to].size());
  std::vector<int> dst = bm->take(to, n);
  for (int64_t i = 0; i < n; ++i) {
    pairs[2 * i] = s->ids[(size_t)i];
    pairs[2 * i + 1] = dst[(size_t)i];
    bm->release(from, s->ids[(size_t)i]);
  }
  s->ids = std::move(dst);
  s->dev = to;
  if (num_pairs) *num_pairs = (int)n;
  return pa_ok();
}

}  // namespace

extern "C" {

int pa_bm_create(int block_size, int num_gpu_blocks, int num_cpu_blocks, pa_bm** out) {
  if (!out) return pa_fail(PA_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (block_size < 1 || num_gpu_blocks < 1 || num_cpu_blocks < 0)
    return pa_fail(PA_ERR_INVALID_ARG, "invalid sizes (block_size %d, gpu %d, cpu %d)", block_size,
                   num_gpu_blocks, num_cpu_blocks);
  pa_bm* bm = new pa_bm;
  bm->bs = block_size;
  const int n[2] = {num_gpu_blocks, num_cpu_blocks};
  for (int d = 0; d < 2; ++d) {
    bm->ref[d].assign((size_t)n[d], 0);
    for (int b = 0; b < n[d]; ++b) bm->free_[d].insert(bm->free_[d].end(), b);
  }
  *out = bm;
  return pa_ok();
}

void pa_bm_destroy(pa_bm* bm) { delete bm; }

int pa_bm_can_allocate(const pa_bm* bm, int num_tokens) {
  if (!bm) return -pa_fail(PA_ERR_NULL, "manager is NULL");
  if (num_tokens < 0) return -pa_fail(PA_ERR_INVALID_ARG, "num_tokens < 0");
  pa_ok();
  return bm->blocks_needed(num_tokens) <= (int64_t)bm->free_[0].size() ? 1 : 0;
}

int pa_bm_allocate(pa_bm* bm, int seq_id, int num_tokens) {
  if (!bm) return pa_fail(PA_ERR_NULL, "manager is NULL");
  if (seq_id < 0 || num_tokens < 0)
    return pa_fail(PA_ERR_INVALID_ARG, "seq_id %d / num_tokens %d must be >= 0", seq_id, num_tokens);
  if (find(bm, seq_id)) return pa_fail(PA_ERR_INVALID_ARG, "sequence %d exists", seq_id);
  const int64_t need = bm->blocks_needed(num_tokens);
  if (need > (int64_t)bm->free_[0].size())
    return pa_fail(PA_ERR_OUT_OF_BLOCKS, "%lld blocks needed, %zu free", (long long)need,
                   bm->free_[0].size());
  pa_bm::Seq s;
  s.dev = 0;
  s.ids = bm->take(0, need);
  s.tokens = num_tokens;
  bm->seqs.emplace(seq_id, std::move(s));
  return pa_ok();
}

int pa_bm_append_slot(pa_bm* bm, int seq_id, int32_t* slot_block, int32_t* slot_row,
                      int32_t* cow_src, int32_t* cow_dst) {
  if (!bm) return pa_fail(PA_ERR_NULL, "manager is NULL");
  pa_bm::Seq* s = find(bm, seq_id);
  if (!s) return pa_fail(PA_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  if (s->dev != 0) return pa_fail(PA_ERR_INVALID_ARG, "sequence %d is swapped out", seq_id);
  const int row = (int)(s->tokens % bm->bs);
  int src = -1, dst = -1;
  if (row == 0 || bm->ref[0][s->ids.back()] > 1) {
    if (bm->free_[0].empty()) return pa_fail(PA_ERR_OUT_OF_BLOCKS, "no free block");
    const int b = bm->take(0, 1)[0];
    if (row == 0) {
      s->ids.push_back(b);
    } else {                                  // copy-on-write of a shared partial block
      src = s->ids.back();
      dst = b;
      bm->release(0, src);
      s->ids.back() = b;
    }
  }
  s->tokens += 1;
  if (slot_block) *slot_block = s->ids.back();
  if (slot_row) *slot_row = row;
  if (cow_src) *cow_src = src;
  if (cow_dst) *cow_dst = dst;
  return pa_ok();
}

int pa_bm_fork(pa_bm* bm, int parent_id, int child_id) {
  if (!bm) return pa_fail(PA_ERR_NULL, "manager is NULL");
  const pa_bm::Seq* p = find(bm, parent_id);
  if (!p) return pa_fail(PA_ERR_INVALID_ARG, "unknown sequence %d", parent_id);
  if (p->dev != 0) return pa_fail(PA_ERR_INVALID_ARG, "sequence %d is swapped out", parent_id);
  if (child_id < 0 || find(bm, child_id))
    return pa_fail(PA_ERR_INVALID_ARG, "child id %d is negative or exists", child_id);
  pa_bm::Seq c = *p;
  for (int b : c.ids) bm->ref[0][b] += 1;
  bm->seqs.emplace(child_id, std::move(c));
  return pa_ok();
}

int pa_bm_free(pa_bm* bm, int seq_id) {
  if (!bm) return pa_fail(PA_ERR_NULL, "manager is NULL");
  auto it = bm->seqs.find(seq_id);
  if (it == bm->seqs.end()) return pa_fail(PA_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  for (int b : it->second.ids) bm->release(it->second.dev, b);
  bm->seqs.erase(it);
  return pa_ok();
}

int pa_bm_swap_out(pa_bm* bm, int seq_id, int32_t* pairs, int max_pairs, int* num_pairs) {
  return swap(bm, seq_id, 0, pairs, max_pairs, num_pairs);
}

int pa_bm_swap_in(pa_bm* bm, int seq_id, int32_t* pairs, int max_pairs, int* num_pairs) {
  return swap(bm, seq_id, 1, pairs, max_pairs, num_pairs);
}

int pa_bm_num_free_blocks(const pa_bm* bm, int on_cpu) {
  if (!bm) return -pa_fail(PA_ERR_NULL, "manager is NULL");
  return (int)bm->free_[on_cpu ? 1 : 0].size();
}

double pa_bm_usage_ratio(const pa_bm* bm) {
  if (!bm) return -1.0;
  const double n = (double)bm->ref[0].size();
  return 1.0 - (double)bm->free_[0].size() / n;
}

int pa_bm_seq_info(const pa_bm* bm, int seq_id, int* num_tokens, int* num_blocks, int* on_cpu) {
  if (!bm) return pa_fail(PA_ERR_NULL, "manager is NULL");
  const pa_bm::Seq* s = find(bm, seq_id);
  if (!s) return pa_fail(PA_ERR_INVALID_ARG, "unknown sequence %d", seq_id);
  if (num_tokens) *num_tokens = (int)s->tokens;
  if (num_blocks) *num_blocks = (int)s->ids.size();
  if (on_cpu) *on_cpu = s->dev;
  return pa_ok();
}

int pa_bm_refcount(const pa_bm* bm, int block, int on_cpu) {
  if (!bm) return -pa_fail(PA_ERR_NULL, "manager is NULL");
  const int d = on_cpu ? 1 : 0;
  if (block < 0 || block >= (int)bm->ref[d].size())
    return -pa_fail(PA_ERR_INVALID_ARG, "block %d out of range", block);
  return bm->ref[d][block];
}

int pa_bm_fill_batch(const pa_bm* bm, const int32_t* seq_ids, int n, int32_t* block_tables,
                     int max_blocks_per_seq, int32_t* context_lens) {
  if (!bm) return pa_fail(PA_ERR_NULL, "manager is NULL");
  if (n < 0 || max_blocks_per_seq < 1) return pa_fail(PA_ERR_INVALID_ARG, "invalid sizes");
  if (n > 0 && (!seq_ids || !block_tables || !context_lens))
    return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  for (int i = 0; i < n; ++i) {
    const pa_bm::Seq* s = find(bm, seq_ids[i]);
    if (!s) return pa_fail(PA_ERR_INVALID_ARG, "unknown sequence %d", seq_ids[i]);
    if (s->dev != 0) return pa_fail(PA_ERR_INVALID_ARG, "sequence %d is swapped out", seq_ids[i]);
    if ((int64_t)s->ids.size() > max_blocks_per_seq)
      return pa_fail(PA_ERR_INVALID_ARG, "sequence %d has %zu blocks > max_blocks_per_seq %d",
                     seq_ids[i], s->ids.size(), max_blocks_per_seq);
  }
  for (int i = 0; i < n; ++i) {
    const pa_bm::Seq* s = find(bm, seq_ids[i]);
    int32_t* row = block_tables + (size_t)i * max_blocks_per_seq;
    for (int j = 0; j < max_blocks_per_seq; ++j) row[j] = j < (int)s->ids.size() ? s->ids[j] : -1;
    context_lens[i] = (int32_t)s->tokens;
  }
  return pa_ok();
}

int pa_bm_prefix_groups(const pa_bm* bm, const int32_t* seq_ids, int n, int32_t* seq_group,
                        int32_t* group_prefix_len, int* num_groups, int* max_group_size) {
  if (!bm) return pa_fail(PA_ERR_NULL, "manager is NULL");
  if (n < 0) return pa_fail(PA_ERR_INVALID_ARG, "n < 0");
  if (n > 0 && (!seq_ids || !seq_group || !group_prefix_len))
    return pa_fail(PA_ERR_NULL, "a required pointer is NULL");
  std::vector<const pa_bm::Seq*> seqs((size_t)n);
  for (int i = 0; i < n; ++i) {
    seqs[(size_t)i] = find(bm, seq_ids[i]);
    if (!seqs[(size_t)i]) return pa_fail(PA_ERR_INVALID_ARG, "unknown sequence %d", seq_ids[i]);
    if (seqs[(size_t)i]->dev != 0)
      return pa_fail(PA_ERR_INVALID_ARG, "sequence %d is swapped out", seq_ids[i]);
  }
  auto full = [&](int i) { return (size_t)(seqs[(size_t)i]->tokens / bm->bs); };
  // Members of each group keyed by the first full block, in order of first
  // appearance.
  std::unordered_map<int, size_t> key_pos;
  std::vector<std::vector<int>> cand;
  for (int i = 0; i < n; ++i) {
    seq_group[i] = -1;
    if (full(i) == 0) continue;
    const int key = seqs[(size_t)i]->ids[0];
    auto it = key_pos.find(key);
    if (it == key_pos.end()) {
      key_pos.emplace(key, cand.size());
      cand.push_back({i});
    } else {
      cand[it->second].push_back(i);
    }
  }
  int groups = 0, largest = 1;
  for (const auto& members : cand) {
    if (members.size() < 2) continue;
    size_t run = full(members[0]);
    for (int i : members) run = std::min(run, full(i));
    const auto& lead = seqs[(size_t)members[0]]->ids;
    size_t k = 0;
    while (k < run) {
      bool same = true;
      for (int i : members) same = same && seqs[(size_t)i]->ids[k] == lead[k];
      if (!same) break;
      ++k;
    }
    for (int i : members) seq_group[i] = groups;
    group_prefix_len[groups] = (int32_t)(k * (size_t)bm->bs);
    ++groups;
    largest = std::max(largest, (int)members.size());
  }
  if (num_groups) *num_groups = groups;
  if (max_group_size) *max_group_size = largest;
  return pa_ok();
}

}  // extern "C"
