// Layout of the split-K workspace: host-only arithmetic, shared by the
// argument checks (pa_api.cpp: the size a caller must provide) and the
// launches (pa_kernels.hip: where each part starts).
#include "pa_launch.h"

namespace pa {

namespace {
size_t up256(size_t x) { return (x + 255) / 256 * 256; }
}  // namespace

// Each part starts on a 256-byte boundary:
//   acc     [B][Hq][Pmax][D] fp32, then (m, l) [B][Hq][Pmax] as fp32 pairs
//   plan    unit count and split count (256 bytes), unit records
//           [(G + B) * Pmax] of 32 bytes, split list [B] of (sequence,
//           partitions) int pairs
//   with prompt groups: member records [B] of 16 bytes, then the plan's
//   scratch: arrival [2B], group_fill [G], group_start [G + 1], group_lp [G].
// num_groups < 0: a plain split-K call, no group tables.
WsLayout ws_layout(int num_seqs, int num_heads, int head_dim, int max_partitions,
                   int num_groups) {
  const bool tables = num_groups >= 0;
  if (num_groups < 0) num_groups = 0;
  WsLayout w;
  const size_t slots = (size_t)num_seqs * num_heads * max_partitions;
  w.max_units = (size_t)(num_groups + num_seqs) * max_partitions;
  w.ml = slots * head_dim * sizeof(float);
  w.n_units = up256(w.ml + slots * 2 * sizeof(float));
  w.units = w.n_units + 256;
  w.split = up256(w.units + w.max_units * kUnitRecordBytes);
  w.minfo = up256(w.split + (size_t)num_seqs * 2 * sizeof(int));
  w.arrival = up256(w.minfo + (size_t)num_seqs * 4 * sizeof(int));
  w.group_fill = up256(w.arrival + (size_t)num_seqs * 2 * sizeof(int));
  w.group_start = up256(w.group_fill + (size_t)num_groups * sizeof(int));
  w.group_lp = up256(w.group_start + (size_t)(num_groups + 1) * sizeof(int));
  w.total = up256(w.group_lp + (size_t)num_groups * sizeof(int));
  if (!tables) w.total = w.minfo;
  return w;
}

size_t splitk_workspace_bytes(int num_seqs, int num_heads, int head_dim, int max_partitions,
                              int num_groups) {
  return ws_layout(num_seqs, num_heads, head_dim, max_partitions, num_groups).total;
}

}  // namespace pa
