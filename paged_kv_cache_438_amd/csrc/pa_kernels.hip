// HIP kernels for paged KV-cache decode attention on CDNA4 (gfx950).
//
// What is computed follows the pages' description of paged attention: K and V
// of a sequence live in fixed-size blocks of a shared pool, a per-sequence
// block table lists them in logical order, and attention is
// softmax(q K^T * scale) V over the concatenation of those blocks
// ("IO-5 vLLM Paged Attention", section 3 "KV Cache Paging structure" and
// section 4 "Attention computation").  The pages name a CUDA kernel that reads
// the table and combines the scattered blocks ("vLLM's efficiency secret:
// PagedAttention and dynamic memory management", section on using the KV
// cache like virtual memory) but give no design for it; everything below is
// designed for gfx950.
//
// Mapping onto the hardware
// -------------------------
// A token row of one head is head_dim * elem bytes (256 B for d=128 fp16/bf16
// and for d=64 fp32).  A wave64 reads it with one 16-byte load per lane:
// LPR = row_bytes/16 lanes share a row ("row group"), and one wave-wide load
// covers RPL = 64/LPR consecutive token rows.  A wave consumes 16 tokens per
// step with NL = 16/RPL loads of K and NL loads of V, all issued before any
// arithmetic, so every wave keeps 2*NL*1 KiB in flight.
//
// q.k: each lane forms the dot product of its 16-byte slice with the matching
// slice of q (v_dot2_f32_f16 / v_dot2_f32_bf16, fp32 accumulation), and the
// LPR lanes of a row group are summed with DPP moves inside the 16-lane row.
//
// Softmax: each row group keeps its own running maximum m (log2 domain), sum
// l and fp32 accumulator over the tokens it has seen; no cross-lane traffic
// is needed inside the loop.  After the loop the row groups of a wave, then
// the waves of a workgroup (through LDS), are merged with the rule
//   m = max(m1, m2), l = l1*2^(m1-m) + l2*2^(m2-m), acc likewise,
// which is the same rescaling the split-K reduce applies across partitions.
//
// Tail and contract handling: a step that runs past the end of its token
// range reads the last valid row instead (so it never touches rows past the
// sequence's length or table entries past its last block) and its scores are
// set to -inf, giving exactly zero weight.  Lengths or block ids outside the
// documented contract make the output NaN instead of faulting.
//
// Kernels in this file
// --------------------
// k_decode       the vector-ALU decode described above (MHA, fp32, and
//                grouped heads under the VALU-only flag).
// k_decode_mfma  grouped heads on the matrix cores: S^T = K Q^T and
//                O^T = V^T P^T per 16-token step, K/V staged in LDS by
//                direct-to-LDS loads; also every shared-prompt unit, whose
//                columns are the queries of all members of a group.
// k_plan         one workgroup per split call: orders the (sequence or
//                group, partition) units longest first and, for shared
//                prompts, builds the group tables.
// k_reduce       merges a split sequence's partitions in fixed order.
// k_cache_write  the new token's K/V into its slot.
// k_copy_blocks  whole-block copies inside the pools (copy-on-write).
// k_swap_blocks  whole-block moves between the device pools and a pinned
//                host pool through its device mapping.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>
#include <type_traits>

#include "pa_launch.h"

namespace pa {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Finite stand-in for -infinity as the initial running maximum: with it,
// 2^(m_old - m_new) is 1 for two empty states and 0 once a real score
// arrives, and no inf - inf ever occurs.
constexpr float kEmptyMax = -1.0e30f;

template <int DT> struct Elem;
template <> struct Elem<kF32> { static constexpr int bytes = 4; };
template <> struct Elem<kF16> { static constexpr int bytes = 2; };
template <> struct Elem<kBF16> { static constexpr int bytes = 2; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf162_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ half2_t as_h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ bf162_t as_b2(uint32_t u) { return __builtin_bit_cast(bf162_t, u); }

// acc + <16 bytes of a key row, the lane's 16 bytes of q>, in fp32.
template <int DT> __device__ __forceinline__ float dot16(uint4 k, uint4 q, float acc);
template <> __device__ __forceinline__ float dot16<kF16>(uint4 k, uint4 q, float acc) {
  acc = __builtin_amdgcn_fdot2(as_h2(k.x), as_h2(q.x), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(k.y), as_h2(q.y), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(k.z), as_h2(q.z), acc, false);
  acc = __builtin_amdgcn_fdot2(as_h2(k.w), as_h2(q.w), acc, false);
  return acc;
}
template <> __device__ __forceinline__ float dot16<kBF16>(uint4 k, uint4 q, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(k.x), as_b2(q.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(k.y), as_b2(q.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(k.z), as_b2(q.z), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(as_b2(k.w), as_b2(q.w), acc, false);
  return acc;
}
template <> __device__ __forceinline__ float dot16<kF32>(uint4 k, uint4 q, float acc) {
  acc = fmaf(__uint_as_float(k.x), __uint_as_float(q.x), acc);
  acc = fmaf(__uint_as_float(k.y), __uint_as_float(q.y), acc);
  acc = fmaf(__uint_as_float(k.z), __uint_as_float(q.z), acc);
  acc = fmaf(__uint_as_float(k.w), __uint_as_float(q.w), acc);
  return acc;
}

// acc[0..EPL) += p * (16 bytes of a value row), fp32.
template <int DT> struct Axpy;
template <> struct Axpy<kF16> {
  static __device__ __forceinline__ void run(float* acc, float p, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2_t h = as_h2(w[i]);
      acc[2 * i] = fmaf(p, (float)h.x, acc[2 * i]);
      acc[2 * i + 1] = fmaf(p, (float)h.y, acc[2 * i + 1]);
    }
  }
};
template <> struct Axpy<kBF16> {
  static __device__ __forceinline__ void run(float* acc, float p, uint4 v) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] = fmaf(p, __uint_as_float(w[i] << 16), acc[2 * i]);
      acc[2 * i + 1] = fmaf(p, __uint_as_float(w[i] & 0xffff0000u), acc[2 * i + 1]);
    }
  }
};
template <> struct Axpy<kF32> {
  static __device__ __forceinline__ void run(float* acc, float p, uint4 v) {
    acc[0] = fmaf(p, __uint_as_float(v.x), acc[0]);
    acc[1] = fmaf(p, __uint_as_float(v.y), acc[1]);
    acc[2] = fmaf(p, __uint_as_float(v.z), acc[2]);
    acc[3] = fmaf(p, __uint_as_float(v.w), acc[3]);
  }
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Inclusive prefix sum over the 64 lanes of a wave: within each 16-lane DPP
// row shift-and-add by 1, 2, 4 and 8 (lanes without a source add 0), then
// carry row 0's total into row 1 and row 2's into row 3 (row_bcast:15), and
// rows 0-1's total into rows 2-3 (row_bcast:31).
__device__ __forceinline__ int wave_inclusive_sum(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);   // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);   // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);   // row_bcast:31
  return v;
}

// Sum over the LPR consecutive lanes of a row group; every lane of the group
// receives the total.  Inside a 16-lane DPP row: swap neighbours, swap pairs,
// mirror halves of 8, mirror the row of 16; groups of 32 add the other row.
template <int LPR>
__device__ __forceinline__ float row_group_sum(float x) {
  x += dpp_f32<0xB1>(x);                       // quad_perm [1,0,3,2]
  x += dpp_f32<0x4E>(x);                       // quad_perm [2,3,0,1]
  if constexpr (LPR >= 8) x += dpp_f32<0x141>(x);   // row_half_mirror
  if constexpr (LPR >= 16) x += dpp_f32<0x140>(x);  // row_mirror
  if constexpr (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

// 16-byte loads of K/V data.  Streaming loads carry the non-temporal hint:
// each block is read by one sequence once per call, so keeping it in L2 or
// the Infinity Cache only displaces other lines.  When blocks are shared by
// several sequences (aliased table entries) the plain, cached load is used.
__device__ __forceinline__ uint4 ld16_stream(const uint8_t* p) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 ld16_cached(const uint8_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}
template <bool NT>
__device__ __forceinline__ uint4 ld16(const uint8_t* p) {
  if constexpr (NT) return ld16_stream(p);
  else return ld16_cached(p);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <int DT> __device__ __forceinline__ void store_elem(void* out, size_t i, float v);
template <> __device__ __forceinline__ void store_elem<kF32>(void* out, size_t i, float v) {
  static_cast<float*>(out)[i] = v;
}
template <> __device__ __forceinline__ void store_elem<kF16>(void* out, size_t i, float v) {
  static_cast<_Float16*>(out)[i] = (_Float16)v;   // round to nearest even
}
template <> __device__ __forceinline__ void store_elem<kBF16>(void* out, size_t i, float v) {
  static_cast<uint16_t*>(out)[i] = f32_to_bf16_rne(v);
}

// One unit of work as the split-K plan lists it (32 bytes, read with one
// scalar load): everything a partition workgroup needs before its first
// table lookup, so that it reaches its first K/V load in three dependent
// memory accesses (the record, the table, the data).
//   s      sequence (>= 0), or -(group + 1) for a partition of a group's
//          shared prompt (sharing-aware decode)
//   pf     partition slot in the low 24 bits, plus kUnit* flags
//   tb, te token range [tb, te) of the unit's main stream
//   first, cnt, lp, ts  (prompt units) the group's members in the member
//          list, its prompt length, and a member whose table supplies the
//          prompt's blocks
struct __attribute__((aligned(16))) URec {
  int s, pf, tb, te, first, cnt, lp, ts;
};
constexpr int kPartMask = (1 << 24) - 1;
constexpr int kUnitDirect = 1 << 24;   // the sequence's only partition: write the output row
constexpr int kUnitBad = 1 << 25;      // out-of-contract sequence: a NaN output row
constexpr int kUnitTail = 1 << 26;     // a group's last prompt partition: absorbed own tokens
// A member of a prompt group, in the group's member order (16 bytes):
// {sequence, absorbed own tokens [y, z) (empty if none), kUnitDirect |
// kUnitBad}.

// Unsigned division by a divisor d fixed at launch, for numerators below
// 2^31: with l = ceil(log2 d) and m = ceil(2^(31+l) / d), floor(x / d) =
// (x * m) >> (31 + l) (the rounding error of m stays below 1/d for such x).
// The host fills it (set_divisor).
struct Divisor {
  uint32_t m;
  int shift;
  __device__ __forceinline__ int div(int x) const {
    return (int)(((uint64_t)(uint32_t)x * m) >> shift);
  }
};

// Plan data the partition launches only read, reached through the constant
// address space so that uniform loads of it stay scalar.
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef const i32x4_t __attribute__((address_space(4)))* const_i32x4_ptr;
typedef const int __attribute__((address_space(4)))* const_int_ptr;

struct KArgs {
  void* out;
  const uint8_t* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  // The new token's rows [B][Hkv][D] when the single-pass launch also writes
  // them (nullptr otherwise): see k_decode's FUSED.
  const uint8_t* k_new;
  const uint8_t* v_new;
  float* ws_acc;        // [B][Hq][max_parts][D]
  float2* ws_ml;        // [B][Hq][max_parts] of (max, sum)
  const int* n_units;   // split-K plan: number of units, then of sequences to merge
  const URec* urecs;    // split-K plan: the units, longest first (nullptr: single pass)
  const int2* split;    // split-K plan: (sequence, partitions) of the sequences to merge
  const int4* minfo;    // split-K plan: members of the prompt groups
  // Sharing-aware decode, read by the plan only (nullptr otherwise): the
  // group of each sequence (-1: none) and each group's shared prompt length.
  const int32_t* seq_group;
  const int32_t* group_prefix;
  int num_groups;
  int num_seqs, num_heads, num_kv_heads, bs_log2, max_blocks, num_blocks;
  int max_len;          // longest valid context: max_blocks << bs_log2, or a contiguous cache's rows
  int group;            // query heads per KV head
  int chunks;           // column chunks (matrix cores) or head chunks (vector ALUs) per KV head
  int part_tokens;      // P
  Divisor part_div;     // division by P
  int members_chunk;    // most members one column chunk of 16 holds
  int max_parts;
  int grid_units;       // units one pass of the grid covers
  int max_units;        // capacity of the unit list
  int xcd_heads;        // consecutive workgroups of a unit per XCD (xcd_group)
  float scale_log2;     // scale * log2(e)
};

// Partition layout of one sequence, as the plan derives it.  Without a
// prompt group, tokens [0, L) are cut into partitions of P tokens.  A
// sequence whose group shares a prompt of Lp tokens (a multiple of the block
// size, the same blocks at the head of every member's table) has the
// prompt's partitions first -- they are computed once for the whole group.
// Its own tokens [Lp, L) follow in partitions of P, unless they are few
// enough to be absorbed into the group's last prompt partition: at most
// P / m tokens, where m bounds the members one column chunk holds, so that
// partition never streams more than P prompt tokens plus P own tokens.  A
// length outside [0, max_blocks * bs], or needing more partitions than the
// grid holds, is a contract violation: no partitions and a NaN output row.
struct SeqLayout {
  int len, lp, np_pre, nparts;
  bool bad, absorbed;
};
// Layout from a sequence's length and group (-1: none); for a group in
// range, lp_g is its prompt length and cnt its member count.  absorb_max[m]
// = P / max(1, m) for m <= members_chunk, the most own tokens a member may
// bring to its group's last prompt partition.
__device__ __forceinline__ SeqLayout layout_of(const KArgs& a, int len, int gi, int lp_g, int cnt,
                                               const int* absorb_max) {
  SeqLayout r;
  r.len = len;
  r.lp = 0;
  r.absorbed = false;
  bool bad = r.len < 0 || r.len > a.max_len;
  if (a.seq_group != nullptr) {
    if (gi >= a.num_groups || gi < -1) bad = true;
    else if (gi >= 0) r.lp = lp_g;
    if (r.lp < 0 || r.lp > r.len || (r.lp & ((1 << a.bs_log2) - 1)) != 0) bad = true;
  }
  if (bad) { r.len = 0; r.lp = 0; }
  r.np_pre = a.part_div.div(r.lp + a.part_tokens - 1);
  if (r.lp > 0) r.absorbed = r.len - r.lp <= absorb_max[min(cnt, a.members_chunk)];
  r.nparts = r.np_pre + (r.absorbed ? 0 : a.part_div.div(r.len - r.lp + a.part_tokens - 1));
  if (r.nparts > a.max_parts) {
    bad = true;
    r.len = r.lp = r.np_pre = r.nparts = 0;
    r.absorbed = false;
  }
  r.bad = bad;
  return r;
}

// The dispatcher hands workgroup i to XCD i % 8.  In plain order, with H
// workgroups (KV heads x chunks) per unit, XCD x would read head tiles x,
// x+8, x+16, ... of every block it touches: tiles a fixed stride apart.
// xcd_group renumbers the workgroups so that each XCD takes c consecutive
// head tiles of a unit at a time: the units' groups of c heads are dealt to
// the XCDs in turn, in unit order, so every XCD reads contiguous stretches of
// c tiles and the longest-first order of a split-K plan is kept up to groups
// of c units.  The host picks c (1: plain order).  A bijection on
// [0, gridDim.x) when c divides H and 8c divides the grid.
__device__ __forceinline__ int xcd_group(int i, int H, int c) {
  if (c <= 1) return i;
  const int x = i % 8, j = i / 8;
  const int grp = (j / c) * 8 + x;            // global index of the c-head group
  const int per_unit = H / c;
  return (grp / per_unit) * H + (grp % per_unit) * c + j % c;
}

// Position of a workgroup: its KV head g, chunk ch and first unit u0.
struct WgPos {
  int ch, g, u0;
};
__device__ __forceinline__ WgPos wg_pos(const KArgs& a) {
  int wg = xcd_group(blockIdx.x, a.chunks * a.num_kv_heads, a.xcd_heads);
  WgPos w;
  w.ch = wg % a.chunks;  wg /= a.chunks;
  w.g = wg % a.num_kv_heads;
  w.u0 = wg / a.num_kv_heads;
  return w;
}

// The units of a workgroup whose first unit is u0.  The grid covers
// grid_units units per pass, taken in the plan's longest-first order by the
// dispatcher; later passes go in snake order (pass 1 gives unit 2W-1-u0 to
// workgroup u0, pass 2 unit 2W+u0, ...), so that the workgroups whose first
// units were the shortest take the next longest.  The first record comes
// with the unit count, which is kept; each later record is fetched while the
// unit before it runs (prefetch(), a load into lanes 0..7 issued before that
// unit's first K/V load, and take() after its epilogue).  Without a plan
// (single pass) unit u0 is sequence u0, whole.
struct UnitCursor {
  int u0, it, n;
  URec r;

  __device__ __forceinline__ int index(int k) const {
    const int W = grid_units_;
    return k * W + ((k & 1) ? W - 1 - u0 : u0);
  }
  int grid_units_;

  // The first unit; false if there is none.  PLAN: whether the launch has a
  // unit list (split-K) or one unit per sequence (single pass).
  template <bool PLAN>
  __device__ __forceinline__ bool first(const KArgs& a, int u0_) {
    u0 = u0_;
    it = 0;
    grid_units_ = a.grid_units;
    if (!PLAN) {
      n = 1;
      const int len = a.lens[u0];
      const bool bad = len < 0 || len > a.max_len;
      r.s = u0;
      r.pf = kUnitDirect | (bad ? kUnitBad : 0);
      r.tb = 0;
      r.te = bad ? 0 : len;
      r.first = r.cnt = r.lp = 0;
      r.ts = u0;
      return true;
    }
    n = *(const_int_ptr)a.n_units;
    const const_i32x4_ptr rec = (const_i32x4_ptr)a.urecs + 2 * min(u0, a.max_units - 1);
    const i32x4_t w0 = rec[0], w1 = rec[1];
    r.s = w0.x; r.pf = w0.y; r.tb = w0.z; r.te = w0.w;
    r.first = w1.x; r.cnt = w1.y; r.lp = w1.z; r.ts = w1.w;
    return u0 < n;
  }
  // Whether the workgroup has a unit after the current one.
  __device__ __forceinline__ bool has_next(const KArgs& a) const {
    return a.urecs != nullptr && index(it + 1) < n;
  }
  // Word `lane` (< 8) of the next unit's record, loaded now.
  __device__ __forceinline__ int prefetch(const KArgs& a, int lane) const {
    if (!has_next(a) || lane >= 8) return 0;
    return reinterpret_cast<const int*>(a.urecs)[8 * index(it + 1) + lane];
  }
  // Move to the next unit, whose record `words` holds in lanes 0..7.
  __device__ __forceinline__ void take(int words) {
    ++it;
    r.s = __builtin_amdgcn_readlane(words, 0);
    r.pf = __builtin_amdgcn_readlane(words, 1);
    r.tb = __builtin_amdgcn_readlane(words, 2);
    r.te = __builtin_amdgcn_readlane(words, 3);
    r.first = __builtin_amdgcn_readlane(words, 4);
    r.cnt = __builtin_amdgcn_readlane(words, 5);
    r.lp = __builtin_amdgcn_readlane(words, 6);
    r.ts = __builtin_amdgcn_readlane(words, 7);
  }
};

// One query column of a matrix-core workgroup: whose query it is, which
// partition slot of that sequence it fills, and whether it writes the output
// directly (the sequence has a single partition).
struct Col {
  int seq, head, part;
  bool valid, direct, bad;
};
// Column n of chunk ch of a unit: for a prompt unit, member cc / G of the
// group at query head g*G + cc % G (cc = 16 ch + n); otherwise query head
// g*G + cc of the unit's sequence.
__device__ __forceinline__ Col column_of(const KArgs& a, const URec& r, int g, int ch, int ncols,
                                         int n) {
  Col c;
  const int cc = ch * 16 + n;
  c.part = r.pf & kPartMask;
  if (r.s < 0) {
    const int mi = cc / a.group;
    c.valid = n < ncols && mi < r.cnt;
    const int4 m = c.valid ? a.minfo[r.first + mi] : make_int4(0, 0, 0, kUnitBad);
    c.seq = m.x;
    c.head = g * a.group + cc % a.group;
    c.bad = (m.w & kUnitBad) != 0;
    c.valid = c.valid && !c.bad;       // an out-of-contract member writes its NaN row itself
    c.direct = (m.w & kUnitDirect) != 0;
  } else {
    c.valid = n < ncols;
    c.seq = r.s;
    c.head = g * a.group + cc;
    c.bad = (r.pf & kUnitBad) != 0;
    c.direct = (r.pf & kUnitDirect) != 0;
  }
  return c;
}

// Software pipeline over a wave's nk steps with two register buffers: the
// loads of step k+1 are issued before step k is computed.  The steady-state
// body issues its loads unconditionally, so the wait the compiler places
// before each compute covers only the older buffer's loads and the newer
// ones stay in flight.
// A scheduling barrier after each batch of loads keeps the compiler from
// sinking them below the compute to shorten register live ranges.
template <typename Buf, typename LoadF, typename ComputeF>
__device__ __forceinline__ void run_pipeline(int nk, LoadF&& load, ComputeF&& compute) {
  if (nk <= 0) return;
  Buf A, B;
  load(0, A);
  int k = 0;
  for (; k + 2 < nk; k += 2) {
    load(k + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(k, A);
    load(k + 2, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(k + 1, B);
  }
  if (k + 1 < nk) {
    load(k + 1, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(k, A);
    compute(k + 1, B);
  } else {
    compute(k, A);
  }
}

// The same with three register buffers: steps k+1 and k+2 are in flight
// while step k is computed (twice the bytes in flight per wave, for kernels
// whose register use allows few waves per CU).  The last two to four steps
// run as straight-line code.
template <typename Buf, typename LoadF, typename ComputeF>
__device__ __forceinline__ void run_pipeline3(int nk, LoadF&& load, ComputeF&& compute) {
  if (nk <= 0) return;
  Buf A, B, C;
  load(0, A);
  if (nk == 1) {
    compute(0, A);
    return;
  }
  load(1, B);
  int k = 0;
  for (; k + 4 < nk; k += 3) {        // entry: steps k (A) and k+1 (B) issued
    load(k + 2, C);
    __builtin_amdgcn_sched_barrier(0);
    compute(k, A);
    load(k + 3, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(k + 1, B);
    load(k + 4, B);
    __builtin_amdgcn_sched_barrier(0);
    compute(k + 2, C);
  }
  const int rest = nk - k;            // 2, 3 or 4 steps left, k and k+1 issued
  if (rest == 2) {
    compute(k, A);
    compute(k + 1, B);
  } else if (rest == 3) {
    load(k + 2, C);
    __builtin_amdgcn_sched_barrier(0);
    compute(k, A);
    compute(k + 1, B);
    compute(k + 2, C);
  } else {
    load(k + 2, C);
    __builtin_amdgcn_sched_barrier(0);
    compute(k, A);
    load(k + 3, A);
    __builtin_amdgcn_sched_barrier(0);
    compute(k + 1, B);
    compute(k + 2, C);
    compute(k + 3, A);
  }
}

// Where the decode kernels find token t of sequence s, KV head g:
//  - kSmallPages: blocks of fewer than 16 tokens; row t % bs of block
//    table[s][t / bs], looked up for every row;
//  - kBigPages: blocks of 16 tokens or more, so a 16-token step lies in one
//    block, looked up once per step;
//  - kContiguous: no table; row t of a region of max_len rows that sequence
//    s owns per KV head, [num_seqs][num_kv_heads][max_len][head_dim] -- the
//    preallocated contiguous cache that paging replaces.  The "block" of
//    every step is the sequence itself.
enum KvLayout { kSmallPages = 0, kBigPages = 1, kContiguous = 2 };

// Block ids of the steps a wave walks, fetched one step ahead of their use.
// Blocks of at least 16 tokens: a 16-token step lies in one block, whose id is
// a wave-uniform scalar load.  Smaller blocks: every lane looks up the block
// of each of its NR rows (vector loads).
template <bool BIG_BLOCKS, int NR>
struct BlockIds {
  int cur[BIG_BLOCKS ? 1 : NR];
  int nxt[BIG_BLOCKS ? 1 : NR];
};

// Register buffers of the vector-ALU kernel's pipeline (2 or 3).
#ifndef PA_VALU_STAGES
#define PA_VALU_STAGES 2
#endif
// Waves per workgroup of the vector-ALU kernel's single pass with one head
// per wave.
#ifndef PA_VALU_SINGLE_WAVES
#define PA_VALU_SINGLE_WAVES 16
#endif

// One workgroup = (KV head g, chunk of GW query heads) of one unit per pass:
// a whole sequence (single pass, PLAN false: one unit per workgroup), or a
// partition of the split-K plan (PLAN true: the workgroup takes units in
// snake order).  Its W waves take the unit's 16-token steps round-robin.
// FUSED (single pass, blocks of 16 tokens or more): the launch also stores
// each sequence's new token.  Row L-1 is then read from k_new / v_new, which
// hold the bytes the store puts in the pool, so no workgroup waits for
// another's store and the arithmetic is that of a decode after the write.
template <int DT, int D, int W, int GW, int LAYOUT, bool NT, bool PLAN, bool FUSED = false>
__global__ __launch_bounds__(W * 64) void k_decode(const KArgs a) {
  static_assert(!FUSED || (!PLAN && LAYOUT == kBigPages), "fused write: single pass, big pages");
  constexpr bool BIG_BLOCKS = LAYOUT != kSmallPages;
  constexpr bool CONTIG = LAYOUT == kContiguous;
  constexpr int EB = Elem<DT>::bytes;
  constexpr int ROWB = D * EB;           // bytes per token row of one head
  constexpr int LPR = ROWB / 16;         // lanes per row
  constexpr int RPL = 64 / LPR;          // rows per wave-wide load
  constexpr int NL = 16 / RPL;           // loads per 16-token step
  constexpr int EPL = 16 / EB;           // elements per lane slice
  static_assert(LPR >= 4 && LPR <= 32 && RPL * LPR == 64 && NL * RPL == 16, "row shape");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane / LPR;              // row group
  const int c = lane % LPR;              // 16-byte slice within the row

  const WgPos pos = wg_pos(a);
  const int ch = pos.ch, g = pos.g;
  UnitCursor cur;
  for (bool more = cur.first<PLAN>(a, pos.u0); more;) {
    const URec ur = cur.r;
    const int next_rec = PLAN ? cur.prefetch(a, lane) : 0;   // before this unit's first K/V load
    const int s = ur.s, p = ur.pf & kPartMask;
    const bool direct = (ur.pf & kUnitDirect) != 0;   // the only partition writes the output itself
    const bool ubad = (ur.pf & kUnitBad) != 0;
    const int t_begin = ur.tb;
    const int t_end = ur.te;
    const int nsteps = t_end > t_begin ? (t_end - t_begin + 15) >> 4 : 0;

    const int h0 = g * a.group + ch * GW;
    uint4 qv[GW];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh)
      qv[hh] = *reinterpret_cast<const uint4*>(
          a.q + ((size_t)(s * a.num_heads + h0 + hh) * D) * EB + c * 16);

    float m[GW], l[GW], acc[GW][EPL];
#pragma unroll
    for (int hh = 0; hh < GW; ++hh) {
      m[hh] = kEmptyMax;
      l[hh] = 0.f;
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc[hh][e] = 0.f;
    }

    // One (block, head) tile; in a contiguous cache, a sequence's rows of one head.
    const int bs_mask = CONTIG ? -1 : (1 << a.bs_log2) - 1;
    const size_t tile_bytes = CONTIG ? (size_t)ROWB * a.max_len : (size_t)ROWB << a.bs_log2;
    const size_t block_bytes = tile_bytes * a.num_kv_heads;
    const int32_t* trow = CONTIG ? nullptr : a.tables + (size_t)s * a.max_blocks;
    bool bad_block = false;

    // FUSED: this lane's slice of the new token's K and V rows.  The last
    // wave of the sequence's first head chunk (it has the fewest steps when
    // they do not divide evenly) loads them now and stores them into the
    // pool after its steps, so no wave waits for them (the same slot and the
    // same skips as k_cache_write).
    const uint8_t* kn_row = nullptr;
    const uint8_t* vn_row = nullptr;
    const bool writer = FUSED && ch == 0 && wave == W - 1 && r == 0 && t_end >= 1;
    uint4 kn_val = make_uint4(0, 0, 0, 0), vn_val = kn_val;
    size_t kn_off = 0;
    bool kn_store = false;
    if constexpr (FUSED) {
      const size_t nrow = ((size_t)s * a.num_kv_heads + g) * ROWB + c * 16;
      kn_row = a.k_new + nrow;
      vn_row = a.v_new + nrow;
      if (writer) {
        const int pos = t_end - 1;
        const int phys = trow[pos >> a.bs_log2];
        kn_store = (unsigned)phys < (unsigned)a.num_blocks;
        kn_off = (size_t)(kn_store ? phys : 0) * block_bytes + (size_t)g * tile_bytes +
                 (size_t)(pos & bs_mask) * ROWB + c * 16;
        kn_val = *reinterpret_cast<const uint4*>(kn_row);
        vn_val = *reinterpret_cast<const uint4*>(vn_row);
      }
    }

    // Iteration k of this wave handles the 16-token step starting at step_t0(k).
    const int nk = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;
    auto step_t0 = [&](int k) { return t_begin + ((wave + k * W) << 4); };
    BlockIds<BIG_BLOCKS, NL> ids;
    // Fetch the block ids of step k into ids.nxt.
    auto fetch_ids = [&](int k) {
      const int t0 = step_t0(k);
      if constexpr (CONTIG) {
        ids.nxt[0] = s;
      } else if constexpr (BIG_BLOCKS) {
        ids.nxt[0] = trow[t0 >> a.bs_log2];
      } else {
#pragma unroll
        for (int i = 0; i < NL; ++i)
          ids.nxt[i] = trow[min(t0 + i * RPL + r, t_end - 1) >> a.bs_log2];
      }
    };
    struct Buf { uint4 k[NL], v[NL]; };
    auto load_step = [&](int k, Buf& b) {
      const int t0 = step_t0(k);
#pragma unroll
      for (int i = 0; i < (BIG_BLOCKS ? 1 : NL); ++i) ids.cur[i] = ids.nxt[i];
      fetch_ids(k + 1 < nk ? k + 1 : k);     // unconditional: no branch around loads
      if constexpr (BIG_BLOCKS) {
        int phys = ids.cur[0];
        if ((unsigned)phys >= (unsigned)a.num_blocks) { bad_block = true; phys = 0; }
        const size_t tile = (size_t)phys * block_bytes + (size_t)g * tile_bytes;
        const uint8_t* kb = a.k_pool + tile + (size_t)(t0 & bs_mask) * ROWB + c * 16;
        const uint8_t* vb = a.v_pool + tile + (size_t)(t0 & bs_mask) * ROWB + c * 16;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int dt = min(i * RPL + r, t_end - 1 - t0);   // last valid row past the end
          const uint8_t* kp = kb + dt * ROWB;
          if constexpr (FUSED) kp = t0 + dt == t_end - 1 ? kn_row : kp;   // the new token
          b.k[i] = ld16<NT>(kp);
        }
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int dt = min(i * RPL + r, t_end - 1 - t0);
          const uint8_t* vp = vb + dt * ROWB;
          if constexpr (FUSED) vp = t0 + dt == t_end - 1 ? vn_row : vp;
          b.v[i] = ld16<NT>(vp);
        }
      } else {
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          const int t = min(t0 + i * RPL + r, t_end - 1);
          int ph = ids.cur[i];
          if ((unsigned)ph >= (unsigned)a.num_blocks) { bad_block = true; ph = 0; }
          const size_t off = (size_t)ph * block_bytes + (size_t)g * tile_bytes +
                             (size_t)(t & bs_mask) * ROWB + c * 16;
          b.k[i] = ld16<NT>(a.k_pool + off);
          b.v[i] = ld16<NT>(a.v_pool + off);
        }
      }
    };
    auto compute_step = [&](int k, const Buf& b) {
      const int t0 = step_t0(k);
      float sc[GW][NL];
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const bool valid = t0 + i * RPL + r < t_end;
#pragma unroll
        for (int hh = 0; hh < GW; ++hh) {
          const float z = row_group_sum<LPR>(dot16<DT>(b.k[i], qv[hh], 0.f)) * a.scale_log2;
          sc[hh][i] = valid ? z : -INFINITY;
        }
      }
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
        float mx = sc[hh][0];
#pragma unroll
        for (int i = 1; i < NL; ++i) mx = fmaxf(mx, sc[hh][i]);
        const float mn = fmaxf(m[hh], mx);
        const float alpha = fast_exp2(m[hh] - mn);
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < NL; ++i) {
          sc[hh][i] = fast_exp2(sc[hh][i] - mn);
          ps += sc[hh][i];
        }
        l[hh] = l[hh] * alpha + ps;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[hh][e] *= alpha;
        m[hh] = mn;
      }
#pragma unroll
      for (int i = 0; i < NL; ++i)
#pragma unroll
        for (int hh = 0; hh < GW; ++hh) Axpy<DT>::run(acc[hh], sc[hh][i], b.v[i]);
    };

    if (nk > 0) fetch_ids(0);
#if PA_VALU_STAGES == 3
    run_pipeline3<Buf>(nk, load_step, compute_step);
#else
    run_pipeline<Buf>(nk, load_step, compute_step);
#endif
    if constexpr (FUSED) {
      // The pools are written only here, by the launch that owns them.
      if (writer && kn_store) {
        *reinterpret_cast<uint4*>(const_cast<uint8_t*>(a.k_pool) + kn_off) = kn_val;
        *reinterpret_cast<uint4*>(const_cast<uint8_t*>(a.v_pool) + kn_off) = vn_val;
      }
    }

    // Merge the row groups of this wave.
#pragma unroll
    for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
        const float mo = __shfl_xor(m[hh], off);
        const float lo = __shfl_xor(l[hh], off);
        const float mn = fmaxf(m[hh], mo);
        const float fa = fast_exp2(m[hh] - mn), fb = fast_exp2(mo - mn);
        l[hh] = l[hh] * fa + lo * fb;
#pragma unroll
        for (int e = 0; e < EPL; ++e)
          acc[hh][e] = acc[hh][e] * fa + __shfl_xor(acc[hh][e], off) * fb;
        m[hh] = mn;
      }
    }

    // Merge the waves through LDS.
    __shared__ float s_acc[W][GW][D];
    __shared__ float s_m[W][GW], s_l[W][GW];
    __shared__ int s_bad;
    if (threadIdx.x == 0) s_bad = 0;
    __syncthreads();
    if (bad_block) s_bad = 1;
    if (r == 0) {
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_acc[wave][hh][c * EPL + e] = acc[hh][e];
        if (c == 0) { s_m[wave][hh] = m[hh]; s_l[wave][hh] = l[hh]; }
      }
    }
    __syncthreads();
    const bool poisoned = ubad || s_bad;
    for (int idx = threadIdx.x; idx < GW * D; idx += W * 64) {
      const int hh = idx / D, e = idx % D;
      float M = s_m[0][hh];
#pragma unroll
      for (int w = 1; w < W; ++w) M = fmaxf(M, s_m[w][hh]);
      float lsum = 0.f, asum = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = fast_exp2(s_m[w][hh] - M);
        lsum += s_l[w][hh] * f;
        asum += s_acc[w][hh][e] * f;
      }
      const int h = h0 + hh;
      if (direct) {
        float v = lsum > 0.f ? asum / lsum : 0.f;
        if (poisoned) v = __builtin_nanf("");
        store_elem<DT>(a.out, (size_t)(s * a.num_heads + h) * D + e, v);
      } else {
        const size_t slot = (size_t)(s * a.num_heads + h) * a.max_parts + p;
        if (poisoned) { asum = __builtin_nanf(""); lsum = __builtin_nanf(""); }
        a.ws_acc[slot * D + e] = asum;
        if (e == 0) a.ws_ml[slot] = make_float2(M, lsum);
      }
    }
    if constexpr (!PLAN) break;
    __syncthreads();                       // the merge arrays are reused by the next unit
    more = cur.has_next(a);
    if (more) cur.take(next_rec);
  }
}

// ----------------------------------------------------------------------------
// Grouped-query decode on the matrix cores.
//
// When several query heads share a KV head, q.K^T and p.V are small dense
// contractions: per 16-token step, S^T = K Q^T is (16 tokens x d) . (d x heads)
// and O^T += V^T P^T is (d x 16 tokens) . (16 tokens x heads).  On the VALU
// path every K row needs a 16-lane DPP reduction per query head and every V
// element G fmas; here both products run on MFMA and the VALU only does the
// softmax and one register transpose of V.
//
// Lane layout of a 16x16 MFMA (wave64): operand lane l holds row/column
// l % 16 and the slice of the contraction index owned by lane group
// l / 16; the result lane l holds column l % 16, rows 4*(l/16) .. +3.
//
//  * S^T = K . Q^T with v_mfma_f32_16x16x32 (one per 32 head-dim elements):
//    lane l reads 16 bytes of token l%16 (chunk 4i + l/16 of its row for
//    product i) and the same chunk of query head l%16.  Both operands use the
//    same head-dim order, so the sum is the ordinary dot product.
//  * The result gives lane l the scores of head n = l%16 for tokens
//    4*(l/16) + r, r = 0..3: exactly the operand layout of P^T in the next
//    product, so the softmax weights never move between lanes.
//  * O^T += V^T . P^T with v_mfma_f32_16x16x16 (one per 16 head-dim
//    elements).  V^T's operand wants four consecutive tokens of one head-dim
//    element per lane, but memory holds rows; lane 4q + a of quad q reads 16
//    bytes of token 4*(l/16) + a and the quad transposes its 32-bit words
//    with two DPP butterfly stages, after which each lane holds two head-dim
//    elements for the quad's four tokens (two output tiles).
//  * The weights p are split into a high part (exact in the 16-bit element
//    type) and the remainder, each multiplied with V, so the weights keep
//    about 14 significant bits while the accumulation stays in fp32.
//
// Result lane l, tile 2i+e, register r holds head l%16 at head-dim element
// 32i + 8*(l/16) + 2r + e: each lane owns 8 consecutive elements per i.
// Heads of the 16 columns beyond the group are zero queries; their results
// are discarded.

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int DT> struct Mma;
template <> struct Mma<kBF16> {
  static __device__ __forceinline__ f32x4_t qk(uint4 k, uint4 q, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, k),
                                                   __builtin_bit_cast(bf16x8_t, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint2 v, uint2 p, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(bf16x4_t, v),
                                                     __builtin_bit_cast(bf16x4_t, p), c, 0, 0, 0);
  }
  // Two weights -> packed high parts (bf16 truncation, exact) and packed
  // remainders (bf16 truncation of p - high).
  static __device__ __forceinline__ void split2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    const uint32_t h0 = __float_as_uint(p0) & 0xffff0000u, h1 = __float_as_uint(p1) & 0xffff0000u;
    const uint32_t r0 = __float_as_uint(p0 - __uint_as_float(h0));
    const uint32_t r1 = __float_as_uint(p1 - __uint_as_float(h1));
    hi = __builtin_amdgcn_perm(h1, h0, 0x07060302u);
    lo = __builtin_amdgcn_perm(r1, r0, 0x07060302u);
  }
};
template <> struct Mma<kF16> {
  static __device__ __forceinline__ f32x4_t qk(uint4 k, uint4 q, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, k),
                                                  __builtin_bit_cast(f16x8_t, q), c, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4_t pv(uint2 v, uint2 p, f32x4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, v),
                                                 __builtin_bit_cast(f16x4_t, p), c, 0, 0, 0);
  }
  // fp16 high parts rounded toward zero, then the rounded remainders.
  static __device__ __forceinline__ void split2(float p0, float p1, uint32_t& hi, uint32_t& lo) {
    typedef __fp16 fp16x2_t __attribute__((ext_vector_type(2)));
    const fp16x2_t h = __builtin_amdgcn_cvt_pkrtz(p0, p1);
    const fp16x2_t r = __builtin_amdgcn_cvt_pkrtz(p0 - (float)h.x, p1 - (float)h.y);
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, r);
  }
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, CTRL, 0xF, 0xF, true);
}

// 4x4 transpose of 32-bit words across the lanes of a quad: on entry lane a
// holds words w[0..3]; on exit w[j] is the word a that lane j held.  Stage 1
// swaps the off-diagonal 2x2 blocks between lanes a and a^2, stage 2
// transposes each 2x2 block between lanes a and a^1.
__device__ __forceinline__ void quad_transpose(uint32_t (&w)[4], int a) {
  const bool hi_half = a & 2, odd = a & 1;
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t got = dpp_u32<0x4E>(hi_half ? w[j] : w[2 + j]);   // quad_perm [2,3,0,1]
    if (hi_half) w[j] = got; else w[2 + j] = got;
  }
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t got = dpp_u32<0xB1>(odd ? w[2 * j] : w[2 * j + 1]);  // quad_perm [1,0,3,2]
    if (odd) w[2 * j] = got; else w[2 * j + 1] = got;
  }
}

// K/V reach the matrix-core operands through LDS.  Each wave owns two slots
// of one 16-token step each (K tile then V tile).  Direct-to-LDS loads
// (global_load_lds_dwordx4) fill a slot without passing through registers,
// so both slots can be in flight while the wave computes from registers:
// the bytes in flight per CU are bounded by LDS, not by the register file.
// Every load instruction reads whole rows (LPR lanes per row, 16 bytes
// each), i.e. whole cache lines.  Inside a slot, chunk c of row r is stored
// at position c ^ swz(r): the operand reads below (16 rows at one chunk for
// K, four rows at four chunks for V) then hit 16 distinct bank groups.
//
// The loads go through the compiler builtin (which manages M0) but the LDS
// reads of the slots are written as inline assembly, with explicit waits:
// vmcnt(n) for the slot's loads, lgkmcnt(0) before a slot is refilled.  The
// compiler would otherwise wait for every outstanding direct-to-LDS load
// before any LDS read, which serialises the two slots.
//
// All operand reads of a step and the lgkmcnt(0) that waits for them are one
// asm statement: the compiler takes an asm output as ready when the asm ends,
// so with the wait inside it no use, copy or spill of an operand can be
// placed before the data has arrived.  The outputs are early-clobber: a read
// in flight must not land in a register that a later read of the same
// statement still takes its address from.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
template <int N> struct LdsReads;
template <> struct LdsReads<4> {   // head_dim 64: 2 K + 2 V operands
  static __device__ __forceinline__ void run(u32x4_t (&o)[4], const uint32_t (&ad)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  }
};
template <> struct LdsReads<8> {   // head_dim 128: 4 K + 4 V operands
  static __device__ __forceinline__ void run(u32x4_t (&o)[8], const uint32_t (&ad)[8]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %9\n\t"
        "ds_read_b128 %2, %10\n\t"
        "ds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\t"
        "ds_read_b128 %5, %13\n\t"
        "ds_read_b128 %6, %14\n\t"
        "ds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0]), "=&v"(o[1]), "=&v"(o[2]), "=&v"(o[3]),
          "=&v"(o[4]), "=&v"(o[5]), "=&v"(o[6]), "=&v"(o[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]),
          "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
        : "memory");
  }
};
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

template <bool NT>
__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* lds) {
  // aux bit 1 = slc: the streaming (non-temporal) policy of ld16_stream
  __builtin_amdgcn_global_load_lds(g, lds, 16, 0, NT ? 2 : 0);
}

// The same 16-byte load to LDS through a buffer resource: `rsrc` covers one
// (block, KV head) tile, `off` is the byte offset inside it (out-of-range
// offsets read zeros instead of faulting).
#ifndef PA_MFMA_BUFFER_LDS
#define PA_MFMA_BUFFER_LDS 1
#endif
template <bool NT>
__device__ __forceinline__ void dma16_buf(__amdgpu_buffer_rsrc_t rsrc, int off, uint8_t* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      rsrc, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, NT ? 2 : 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint8_t* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(base), 0, bytes, 0x00020000);
}

// Block tables are read-only for the whole kernel: reading them through the
// constant address space lets wave-uniform lookups stay scalar loads even
// though the inline assembly above is marked as touching memory.
typedef const int32_t __attribute__((address_space(4)))* const_i32_ptr;

// Position of 16-byte chunk c of row r (r < 16) inside a slot row.
template <int D>
__device__ __forceinline__ int swz_pos(int c, int r) {
  if constexpr (D == 128) return c ^ (((r & 3) << 2) | (r >> 2));
  else return c ^ ((r >> 1) & 7);
}

// One workgroup = (KV head g, chunk of up to 16 query columns) of one unit
// per pass: a whole sequence (single pass), or a unit of the split-K plan
// (a partition of a sequence, or of a group's shared prompt for all its
// members), taken in snake order with the next unit's record prefetched.
// Its W waves take the unit's 16-token steps round-robin.
// Dynamic LDS: W * 4 * 16 * D * 2 bytes (two slots of K and V tiles per
// wave), reused after the loop for the merge of the waves.
// Occupancy the register allocation aims at: two waves per SIMD (LDS holds
// two workgroups per CU anyway); it keeps the kernel in VGPRs only.
#ifndef PA_MFMA_WPE
#define PA_MFMA_WPE 2
#endif
template <int DT, int D, int W, int LAYOUT, bool NT>
__global__ __launch_bounds__(W * 64) __attribute__((amdgpu_waves_per_eu(PA_MFMA_WPE)))
void k_decode_mfma(const KArgs a) {
  constexpr bool BIG_BLOCKS = LAYOUT != kSmallPages;
  constexpr bool CONTIG = LAYOUT == kContiguous;
  constexpr int EB = 2;
  constexpr int ROWB = D * EB;
  constexpr int LPR = ROWB / 16;      // lanes (16-byte chunks) per row
  constexpr int RPI = 64 / LPR;       // rows per load instruction
  constexpr int NDMA = 16 / RPI;      // load instructions per 16-row tile
  constexpr int TILE = 16 * ROWB;
  constexpr int SLOT = 2 * TILE;      // K tile, V tile
  constexpr int NI = D / 32;          // K (and V) operands of 16 bytes per lane per step
  constexpr int NTILE = D / 16;       // output tiles of 16 head-dim elements
  static_assert(NI * 32 == D && RPI * ROWB == 1024, "head_dim");
  static_assert(sizeof(URec) == kUnitRecordBytes, "unit record");

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 15;            // head column
  const int lg = lane >> 4;           // lane group: owns tokens 4*lg .. 4*lg+3
  const int qa = lane & 3;            // position in the quad
  const int qb = (lane >> 2) & 3;     // quad index inside the lane group

  const WgPos pos = wg_pos(a);
  const int g = pos.g, ch = pos.ch;
  UnitCursor cur;
  for (bool more = a.urecs != nullptr ? cur.first<true>(a, pos.u0) : cur.first<false>(a, pos.u0);
       more;) {
    const URec ur = cur.r;
    // The next unit's record, in flight before this unit's first K/V load (the
    // explicit vmcnt waits below count only loads issued after it).
    const int next_rec = cur.prefetch(a, lane);
    const bool tail = (ur.pf & kUnitTail) != 0;
    const int nh = min(16, (ur.s < 0 ? ur.cnt : 1) * a.group - ch * 16);   // columns in use
    if (nh > 0) {                                  // else a chunk past this group's members
    const bool ubad = (ur.pf & kUnitBad) != 0;
    const int ts = ur.s < 0 ? ur.ts : ur.s;        // whose table supplies stream 0
    const Col col = column_of(a, ur, g, ch, nh, n);   // this lane's column
    uint4 qv[NI];                                  // Q^T operand, loaded below

    // Token streams of the workgroup, 16-token steps each.  Stream 0 is the
    // unit's token range [tb, te) through the table of sequence ts.  A group's
    // last prompt partition adds one stream per member of the chunk, holding
    // that member's absorbed own tokens through its own table; only that
    // member's columns see them (the others get weight exactly 0).  Lane i
    // describes stream i: first step, token range, sequence, member index (-1:
    // every column).  Global step j goes to wave j % W.
    const int cc0 = ch * 16;
    const int col_mi = (cc0 + n) / a.group;        // member index of this lane's column
    const int cnt0 = ur.te > ur.tb ? (ur.te - ur.tb + 15) >> 4 : 0;   // steps of stream 0
    int st_first = 0, st_tb = 0, st_te = 0, st_seq = ts, st_mi = -1;
    int4 mrec = make_int4(ts, 0, 0, 0);
    if (tail && lane > 0) {
      const int mi_lo = cc0 / a.group;
      const int nm = (cc0 + nh - 1) / a.group - mi_lo + 1;
      if (lane <= nm) {
        st_mi = mi_lo + lane - 1;
        mrec = a.minfo[ur.first + st_mi];          // in flight with the first table lookup
      }
    }
    struct StepAt { int t0, t_end, mi, seq; const_i32_ptr trow; };
    // The stream of a step: stream 0 while the step is within it, else the
    // highest lane whose first step is not after it (streams without steps
    // share the next stream's first step).
    auto step_at = [&](int k) {
      const int j = wave + k * W;
      StepAt r;
      if (j < cnt0 || !tail) {
        r.t0 = ur.tb + (j << 4);
        r.t_end = ur.te;
        r.mi = -1;
        r.seq = ts;
      } else {
        const uint64_t le = __builtin_amdgcn_ballot_w64(st_first <= j);
        const int si = 63 - __builtin_clzll(le);
        r.t0 = __builtin_amdgcn_readlane(st_tb, si) +
               ((j - __builtin_amdgcn_readlane(st_first, si)) << 4);
        r.t_end = __builtin_amdgcn_readlane(st_te, si);
        r.mi = __builtin_amdgcn_readlane(st_mi, si);
        r.seq = __builtin_amdgcn_readlane(st_seq, si);
      }
      if constexpr (!CONTIG) r.trow = (const_i32_ptr)(a.tables + (size_t)r.seq * a.max_blocks);
      return r;
    };
    // Row of the step this lane loads with instruction j (clamped to the last
    // valid row past the end), and its position in the slot row.
    const int lrow = lane / LPR;
    const int lpos = lane % LPR;
    BlockIds<BIG_BLOCKS, NDMA> ids;
    auto fetch_ids = [&](int k) {
      const StepAt st = step_at(k);
      if constexpr (CONTIG) {
        ids.nxt[0] = st.seq;
      } else if constexpr (BIG_BLOCKS) {
        ids.nxt[0] = st.trow[st.t0 >> a.bs_log2];
      } else {
#pragma unroll
        for (int j = 0; j < NDMA; ++j)
          ids.nxt[j] = st.trow[min(st.t0 + j * RPI + lrow, st.t_end - 1) >> a.bs_log2];
      }
    };
    // The block ids of this wave's first step go out with the member records
    // when the step lies in stream 0 (it needs no stream table).
    const bool first_in0 = wave < cnt0;
    if (first_in0) fetch_ids(0);
    int nsteps = cnt0;
    if (tail) {
      if (lane == 0) {
        st_tb = ur.tb;
        st_te = ur.te;
      } else if (st_mi >= 0) {
        st_seq = mrec.x;
        st_tb = mrec.y;                            // empty unless absorbed
        st_te = mrec.z;
      }
      const int cnt = st_te > st_tb ? (st_te - st_tb + 15) >> 4 : 0;
      const int incl = wave_inclusive_sum(cnt);
      st_first = incl - cnt;
      nsteps = __builtin_amdgcn_readlane(incl, 63);
    }
    if (!first_in0 && nsteps > wave) fetch_ids(0);

    extern __shared__ __attribute__((aligned(16))) uint8_t s_dyn[];
    uint8_t* wave_lds = s_dyn + wave * 2 * SLOT;
    const uint32_t wave_lds_addr = (uint32_t)(uintptr_t)wave_lds;

    f32x4_t acc[NTILE];
#pragma unroll
    for (int t = 0; t < NTILE; ++t) acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float m = kEmptyMax, lsum = 0.f;

    const int bs_mask = CONTIG ? -1 : (1 << a.bs_log2) - 1;
    const size_t tile_bytes = CONTIG ? (size_t)ROWB * a.max_len : (size_t)ROWB << a.bs_log2;
    const size_t block_bytes = tile_bytes * a.num_kv_heads;
    bool bad_block = false;

    const int nk = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;
    auto issue = [&](int k, int slot) {
      const StepAt st = step_at(k);
      const int t0 = st.t0, t_end = st.t_end;
#pragma unroll
      for (int i = 0; i < (BIG_BLOCKS ? 1 : NDMA); ++i) ids.cur[i] = ids.nxt[i];
      fetch_ids(k + 1 < nk ? k + 1 : k);
      uint8_t* dst = wave_lds + slot * SLOT;
      if constexpr (BIG_BLOCKS && PA_MFMA_BUFFER_LDS) {
        // One block per step: buffer resources over its K and V tiles.
        int ph = ids.cur[0];
        if ((unsigned)ph >= (unsigned)a.num_blocks) { bad_block = true; ph = 0; }
        const size_t tile = (size_t)ph * block_bytes + (size_t)g * tile_bytes;
        const __amdgpu_buffer_rsrc_t rk = tile_rsrc(a.k_pool + tile, (int)tile_bytes);
        const __amdgpu_buffer_rsrc_t rv = tile_rsrc(a.v_pool + tile, (int)tile_bytes);
#pragma unroll
        for (int j = 0; j < NDMA; ++j) {
          const int row = j * RPI + lrow;
          const int t = min(t0 + row, t_end - 1);
          const int off = (t & bs_mask) * ROWB + swz_pos<D>(lpos, row) * 16;
          dma16_buf<NT>(rk, off, dst + j * 1024);
          dma16_buf<NT>(rv, off, dst + TILE + j * 1024);
        }
      } else {
#pragma unroll
        for (int j = 0; j < NDMA; ++j) {
          const int row = j * RPI + lrow;
          const int t = min(t0 + row, t_end - 1);
          int ph = ids.cur[BIG_BLOCKS ? 0 : j];
          if ((unsigned)ph >= (unsigned)a.num_blocks) { bad_block = true; ph = 0; }
          const size_t off = (size_t)ph * block_bytes + (size_t)g * tile_bytes +
                             (size_t)(t & bs_mask) * ROWB + swz_pos<D>(lpos, row) * 16;
          dma16<NT>(a.k_pool + off, dst + j * 1024);
          dma16<NT>(a.v_pool + off, dst + TILE + j * 1024);
        }
      }
    };
    struct Ops { uint4 k[NI], v[NI]; };
    // Operand reads from a slot, waited for before they are returned: K of
    // row n at chunk 4i + lg; V of row 4*lg + qa at chunk 4i + qb.
    auto read_ops = [&](int slot) {
      const uint32_t base = wave_lds_addr + slot * SLOT;
      const int vr = 4 * lg + qa;
      uint32_t ad[2 * NI];
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        ad[i] = base + n * ROWB + swz_pos<D>(4 * i + lg, n) * 16;
        ad[NI + i] = base + TILE + vr * ROWB + swz_pos<D>(4 * i + qb, vr) * 16;
      }
      u32x4_t r[2 * NI];
      LdsReads<2 * NI>::run(r, ad);
      Ops o;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        o.k[i] = make_uint4(r[i].x, r[i].y, r[i].z, r[i].w);
        o.v[i] = make_uint4(r[NI + i].x, r[NI + i].y, r[NI + i].z, r[NI + i].w);
      }
      return o;
    };
    auto compute_step = [&](int k, const Ops& b) {
      const StepAt st = step_at(k);
      const bool mine = st.mi < 0 || st.mi == col_mi;
      f32x4_t sc = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < NI; ++i) sc = Mma<DT>::qk(b.k[i], qv[i], sc);
      float z[4];
#pragma unroll
      for (int r = 0; r < 4; ++r)
        z[r] = (mine && st.t0 + 4 * lg + r < st.t_end) ? sc[r] * a.scale_log2 : -INFINITY;
      float mx = fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mn = fmaxf(m, mx);
      const float alpha = fast_exp2(m - mn);
      m = mn;
      float pr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) pr[r] = fast_exp2(z[r] - mn);
      lsum = lsum * alpha + ((pr[0] + pr[1]) + (pr[2] + pr[3]));
      if (__builtin_amdgcn_ballot_w64(alpha != 1.f) != 0) {   // wave-uniform skip
#pragma unroll
        for (int t = 0; t < NTILE; ++t) acc[t] *= alpha;
      }
      uint2 phi, plo;
      Mma<DT>::split2(pr[0], pr[1], phi.x, plo.x);
      Mma<DT>::split2(pr[2], pr[3], phi.y, plo.y);
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        uint32_t w[4] = {b.v[i].x, b.v[i].y, b.v[i].z, b.v[i].w};
        quad_transpose(w, qa);
        // tile 2i: low halves (element 2*qa of the chunk), tile 2i+1: high halves
        const uint2 v0 = make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u),
                                    __builtin_amdgcn_perm(w[3], w[2], 0x05040100u));
        const uint2 v1 = make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u),
                                    __builtin_amdgcn_perm(w[3], w[2], 0x07060302u));
        acc[2 * i] = Mma<DT>::pv(v0, phi, acc[2 * i]);
        acc[2 * i] = Mma<DT>::pv(v0, plo, acc[2 * i]);
        acc[2 * i + 1] = Mma<DT>::pv(v1, phi, acc[2 * i + 1]);
        acc[2 * i + 1] = Mma<DT>::pv(v1, plo, acc[2 * i + 1]);
      }
    };

    // Q^T operand: column n's query row, chunk 4i + lg (zero for unused
    // columns).  Its loads go out between the first and second slot's K/V loads,
    // so their latency overlaps the first tile's and waiting for them (vmcnt
    // counts in order) leaves the second slot in flight.
    auto load_q = [&]() {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        qv[i] = make_uint4(0, 0, 0, 0);
        if (col.valid)
          qv[i] = *reinterpret_cast<const uint4*>(
              a.q + ((size_t)(col.seq * a.num_heads + col.head) * D) * EB + (4 * i + lg) * 16);
      }
    };

    // Two slots in flight; a slot is refilled as soon as its operands are in
    // registers.
    if (nk > 0) {
      issue(0, 0);                              // its block ids were fetched above
      load_q();
      if (nk > 1) {
        issue(1, 1);
        wait_vmcnt<2 * NDMA>();
      } else {
        wait_vmcnt<0>();
      }
    } else {
      load_q();
      wait_vmcnt<0>();
    }
#pragma unroll
    for (int i = 0; i < NI; ++i)
      asm volatile("" : "+v"(qv[i].x), "+v"(qv[i].y), "+v"(qv[i].z), "+v"(qv[i].w));
    for (int k = 0; k < nk; ++k) {
      const int slot = k & 1;
      if (k + 1 < nk) wait_vmcnt<2 * NDMA>();   // the younger slot may stay in flight
      else wait_vmcnt<0>();
      const Ops ops = read_ops(slot);           // the slot is read: it may be refilled
      if (k + 2 < nk) issue(k + 2, slot);
      compute_step(k, ops);
    }

    // Sum of weights of head n over the wave's four lane groups.
    lsum += __shfl_xor(lsum, 16);
    lsum += __shfl_xor(lsum, 32);

    // Merge the waves through LDS (the slots are free once every wave is here:
    // each wave's last step waited for all of its loads).
    __syncthreads();
    float* s_acc = reinterpret_cast<float*>(s_dyn);          // [W][nh][D]
    float* s_m = s_acc + (size_t)W * nh * D;                // [W][16]
    float* s_l = s_m + W * 16;                              // [W][16]
    int* s_bad = reinterpret_cast<int*>(s_l + W * 16);
    int* s_col = s_bad + 1;                                 // [16][4]: seq, head, part, flags
    if (threadIdx.x == 0) *s_bad = 0;
    if (threadIdx.x < 16) {
      s_col[4 * n] = col.seq;
      s_col[4 * n + 1] = col.head;
      s_col[4 * n + 2] = col.part;
      s_col[4 * n + 3] = (col.valid ? 1 : 0) | (col.direct ? 2 : 0) | (col.bad ? 4 : 0);
    }
    __syncthreads();
    if (bad_block) *s_bad = 1;
    if (n < nh) {
      float* dst = s_acc + ((size_t)wave * nh + n) * D;
#pragma unroll
      for (int i = 0; i < NI; ++i)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          *reinterpret_cast<float2*>(dst + 32 * i + 8 * lg + 2 * r) =
              make_float2(acc[2 * i][r], acc[2 * i + 1][r]);
      if (lg == 0) { s_m[wave * 16 + n] = m; s_l[wave * 16 + n] = lsum; }
    }
    __syncthreads();
    const bool unit_bad = ubad || *s_bad;
    for (int idx = threadIdx.x; idx < nh * D; idx += W * 64) {
      const int hh = idx / D, e = idx % D;
      const int cflags = s_col[4 * hh + 3];
      if (!(cflags & 1)) continue;
      const int cseq = s_col[4 * hh], chead = s_col[4 * hh + 1], cpart = s_col[4 * hh + 2];
      const bool poisoned = unit_bad || (cflags & 4);
      float M = s_m[hh];
#pragma unroll
      for (int w = 1; w < W; ++w) M = fmaxf(M, s_m[w * 16 + hh]);
      float ls = 0.f, as = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const float f = fast_exp2(s_m[w * 16 + hh] - M);
        ls += s_l[w * 16 + hh] * f;
        as += s_acc[((size_t)w * nh + hh) * D + e] * f;
      }
      if (cflags & 2) {
        float v = ls > 0.f ? as / ls : 0.f;
        if (poisoned) v = __builtin_nanf("");
        store_elem<DT>(a.out, (size_t)(cseq * a.num_heads + chead) * D + e, v);
      } else {
        const size_t slot = (size_t)(cseq * a.num_heads + chead) * a.max_parts + cpart;
        if (poisoned) { as = __builtin_nanf(""); ls = __builtin_nanf(""); }
        a.ws_acc[slot * D + e] = as;
        if (e == 0) a.ws_ml[slot] = make_float2(M, ls);
      }
    }
    __syncthreads();                            // the next unit's loads refill the slots
    }
    more = cur.has_next(a);
    if (more) cur.take(next_rec);
  }
}

struct PArgs {
  KArgs k;              // sizes, lengths and (sharing-aware decode) the caller's groups
  int* n_units;         // [0] units, [1] sequences with several partitions
  URec* urecs;          // [max_units]
  int2* split;          // [num_seqs]: (sequence, partitions) of the sequences to merge
  int4* minfo;          // [num_seqs]: members of the groups, grouped, in sequence order
  int* arrival;         // [2 num_seqs] scratch when the members do not fit in LDS: ranks, members
  int* group_fill;      // [num_groups] scratch when the groups do not fit in LDS
  int* group_start;     // [num_groups + 1] scratch, likewise
  int* group_lp;        // [num_groups] scratch, likewise
  int max_group_size;
};

// Threads of the plan's single workgroup.
#ifndef PA_PLAN_THREADS
#define PA_PLAN_THREADS 256
#endif
constexpr int kPlanThreads = PA_PLAN_THREADS;
static_assert(kPlanThreads % 64 == 0 && kPlanThreads >= 256, "plan workgroup");

// Exclusive prefix sum of n ints (src -> dst, dst[n] = total) by the plan's
// workgroup, kPlanThreads entries at a time.
__device__ __forceinline__ void block_exclusive_scan(const int* src, int* dst, int n, int* s_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  int carry = 0;
  for (int base = 0; base < n; base += kPlanThreads) {
    const int v = base + tid < n ? src[base + tid] : 0;
    const int incl = wave_inclusive_sum(v);
    if (lane == 63) s_tot[wv] = incl;
    __syncthreads();
    int before = carry;
    for (int w = 0; w < wv; ++w) before += s_tot[w];
    if (base + tid < n) dst[base + tid] = before + incl - v;
    int chunk = 0;
    for (int w = 0; w < kPlanThreads / 64; ++w) chunk += s_tot[w];
    __syncthreads();
    carry += chunk;
  }
  if (tid == 0) dst[n] = carry;
}

// Sequences and groups whose data the plan keeps in LDS (about 80 KiB in
// all); beyond these counts it reads and writes global memory instead.
constexpr int kPlanSeqs = 4096;
constexpr int kPlanGroups = 1024;
// Runs of full partitions the plan queues for whole waves to write.
constexpr int kPlanLongRuns = 256;

// A sequence's own tokens in ceil(len / P) parts of equal length (whole
// 16-token steps, at most P tokens, the last holding the rest) rather than
// parts of P tokens and a remainder: the longest units are then no longer
// than they need to be (1: on).
#ifndef PA_BALANCED_PARTS
#define PA_BALANCED_PARTS 1
#endif
// Record i of a run of full partitions starting with record r: partition
// slot + i, token range shifted by i partitions.
__device__ __forceinline__ URec run_record(const URec& r, int i) {
  const int stride = r.te - r.tb;       // every record of a run spans the same tokens
  URec x = r;
  x.pf += i;
  x.tb += i * stride;
  x.te += i * stride;
  return x;
}

// Split-K plan, one workgroup.  Every sequence contributes its own
// partitions (at least one unit, so that empty or out-of-contract sequences
// still write their row); with shared prompts every group also contributes
// the partitions of its prompt, each a single unit for all members.  The
// units are counting-sorted by size into 256 buckets, largest first, so the
// partition kernel's workgroups are dispatched longest first (longest-first
// list scheduling).  The order inside a bucket depends on timing; no result
// does, because every column's arithmetic, the streams of a unit (members
// in ascending sequence order) and the reduce's order are fixed.  Each unit
// is written as a complete record (URec), each member of a group as a
// member record, and each sequence with several partitions as (sequence,
// partitions) for the reduce, so the later launches never read the lengths
// or the groups again.  Lengths, groups and group tables are staged in LDS.
__device__ __forceinline__ void plan_body(const PArgs& pa) {
  __shared__ int hist[257];           // bucket counts, then starts (+ total)
  __shared__ int s_tot[kPlanThreads / 64];
  __shared__ int s_split;             // sequences with more than one partition
  __shared__ int s_len[kPlanSeqs], s_grp[kPlanSeqs], s_rank[kPlanSeqs], s_mem[kPlanSeqs];
  // Prompt groups: each sequence's layout as the member phase computed it,
  // its partitions (-1: out of contract) and prompt length, for the passes.
  __shared__ int s_npc[kPlanSeqs], s_lpc[kPlanSeqs];
  __shared__ int s_gfill[kPlanGroups], s_gstart[kPlanGroups + 1], s_glp[kPlanGroups];
  __shared__ int s_gabs[kPlanGroups];
  __shared__ int s_absorb[17];        // P / max(1, m), m = 0 .. 16
  __shared__ int s_nlong;             // runs of full partitions written by whole waves
  __shared__ URec s_lrec[kPlanLongRuns];
  __shared__ int s_lat[kPlanLongRuns], s_ln[kPlanLongRuns];
  const int tid = threadIdx.x;
  const KArgs a = pa.k;
  const int P = a.part_tokens;
  const int B = a.num_seqs;
  const bool shared = a.seq_group != nullptr;
  const int NG = shared ? a.num_groups : 0;
  const bool lds_groups = NG <= kPlanGroups;
  int* gfill = lds_groups ? s_gfill : pa.group_fill;
  int* gstart = lds_groups ? s_gstart : pa.group_start;
  int* glp = lds_groups ? s_glp : pa.group_lp;
  if (tid < 256) hist[tid] = 0;
  if (tid == 0) { s_split = 0; s_nlong = 0; }
  if (tid <= 16) s_absorb[tid] = P / max(1, tid);
  for (int i = tid; i < NG; i += kPlanThreads) gfill[i] = 0;
  for (int s = tid; s < min(B, kPlanSeqs); s += kPlanThreads) {
    s_len[s] = a.lens[s];
    s_grp[s] = shared ? a.seq_group[s] : -1;
  }
  for (int i = tid; i < NG; i += kPlanThreads) glp[i] = a.group_prefix[i];   // checked below
  __syncthreads();
  auto len_of = [&](int s) { return s < kPlanSeqs ? s_len[s] : a.lens[s]; };
  auto grp_of = [&](int s) { return !shared ? -1 : (s < kPlanSeqs ? s_grp[s] : a.seq_group[s]); };
  auto layout = [&](int s) {
    const int gi = grp_of(s);
    int lp = 0, cnt = 0;
    if (gi >= 0 && gi < NG) {
      lp = glp[gi];
      cnt = gstart[gi + 1] - gstart[gi];
    }
    return layout_of(a, len_of(s), gi, lp, cnt, s_absorb);
  };
  int* members = s_mem;                // members of the groups, in sequence order within each
  int* gabs = lds_groups ? s_gabs : pa.group_fill;   // reuses the member counts' scratch
  if (shared) {
    // Members of each group in ascending sequence order, so which member's
    // own tokens a workgroup streams at which step does not depend on
    // timing.  The rank of a member among its group's is counted without
    // atomics: sequences go kPlanThreads at a time, one wave after another;
    // inside a wave, ballots over the bits of the group index find the lanes
    // of the same group, and the group's count so far (gfill) is read by all
    // of them before the lowest of them adds the wave's share.
    const int lane = tid & 63, wv = tid >> 6;
    const int gbits = NG > 1 ? 32 - __builtin_clz(NG - 1) : 0;
    for (int base = 0; base < B; base += kPlanThreads) {
      const int s = base + tid;
      const int gi = s < B ? grp_of(s) : -1;
      const bool in = gi >= 0 && gi < NG;
      uint64_t same = __builtin_amdgcn_ballot_w64(in);
      for (int b = 0; b < gbits; ++b) {
        const bool bit = (gi >> b) & 1;
        const uint64_t set = __builtin_amdgcn_ballot_w64(bit);
        same &= bit ? set : ~set;
      }
      const int below = __builtin_popcountll(same & ((1ull << lane) - 1));
      for (int w = 0; w < kPlanThreads / 64; ++w) {
        if (wv == w && in) {
          const int before = gfill[gi];
          if (below == 0) gfill[gi] = before + __builtin_popcountll(same);
          if (s < kPlanSeqs) s_rank[s] = before + below;
          else pa.arrival[s] = before + below;
        }
        __syncthreads();
      }
    }
    auto validate_groups = [&]() {
      for (int i = tid; i < NG; i += kPlanThreads) {
        // A prompt that is not whole blocks, longer than a table can hold,
        // cut into more partitions than a sequence may have, or shared by
        // more members than the launch's column chunks cover is out of
        // contract: it is marked invalid (-1), so its members get NaN rows.
        const int cnt = gfill[i];
        const int lp = glp[i];
        const bool ok = cnt <= pa.max_group_size && lp >= 0 &&
                        lp <= a.max_len &&
                        (lp & ((1 << a.bs_log2) - 1)) == 0 && (lp + P - 1) / P <= a.max_parts;
        glp[i] = ok ? lp : -1;
        gabs[i] = 0;
      }
    };
    // In LDS the absorbed-token sums have their own array and are cleared
    // beside the scan; in global memory they reuse the counts, so only after.
    if (lds_groups) validate_groups();
    if (NG <= 64) {                     // group starts: one wave's scan
      if (wv == 0) {
        const int v = lane < NG ? gfill[lane] : 0;
        const int incl = wave_inclusive_sum(v);
        if (lane < NG) gstart[lane] = incl - v;
        if (lane == 63) gstart[NG] = incl;
      }
    } else {
      block_exclusive_scan(gfill, gstart, NG, s_tot);
    }
    __syncthreads();
    if (!lds_groups) {
      validate_groups();
      __syncthreads();
    }
    // Each member at its place: the member list, and its record (sequence,
    // absorbed own tokens, flags); gabs[gi] <- absorbed own tokens of the
    // group per column chunk (at most about P by the absorption bound).
    const int nmem = gstart[NG];
    int* mem = nmem <= kPlanSeqs ? s_mem : pa.arrival + B;
    for (int s = tid; s < B; s += kPlanThreads) {
      const SeqLayout ml = layout(s);
      if (s < kPlanSeqs) {
        s_npc[s] = ml.bad ? -1 : ml.nparts;
        s_lpc[s] = ml.lp;
      }
      const int gi = grp_of(s);
      if (gi < 0 || gi >= NG) continue;
      const int lo = gstart[gi], hi = gstart[gi + 1];
      const int at = lo + (s < kPlanSeqs ? s_rank[s] : pa.arrival[s]);
      mem[at] = s;
      const bool own = ml.absorbed && !ml.bad;
      pa.minfo[at] = make_int4(s, own ? ml.lp : 0, own ? ml.len : 0,
                               (ml.nparts == 1 ? kUnitDirect : 0) | (ml.bad ? kUnitBad : 0));
      if (own) atomicAdd(&gabs[gi], (ml.len - ml.lp) / (((hi - lo) * a.group + 15) / 16));
    }
    members = mem;
    __syncthreads();
  }
  // A sequence's layout in the passes: with prompt groups, from what the
  // member phase kept (a shorter chain of LDS reads than layout()).
  auto seq_layout = [&](int s) {
    if (!shared || s >= kPlanSeqs) return layout(s);
    SeqLayout r;
    const int np = s_npc[s];
    r.bad = np < 0;
    r.nparts = r.bad ? 0 : np;
    r.lp = r.bad ? 0 : s_lpc[s];
    r.len = r.bad ? 0 : s_len[s];
    r.np_pre = a.part_div.div(r.lp + P - 1);
    r.absorbed = false;                 // not needed by the passes
    return r;
  };
  // Units hold up to 2P tokens (a last prompt partition with absorbed own
  // tokens); buckets split [0, 2P] evenly, largest first.
  const float bucket_scale = 128.f / (float)P;
  auto bucket = [&](int size) {
    const int b = (int)((float)(2 * P - size) * bucket_scale);   // only the order depends on it
    return b < 0 ? 0 : (b > 255 ? 255 : b);
  };
  // Prompt partitions of a group: np_pre units, the last holding the rest.
  auto prompt_parts = [&](int gi) {
    const int cnt = gstart[gi + 1] - gstart[gi];
    const int lp = glp[gi];
    if (cnt == 0 || lp <= 0) return 0;
    return (lp + P - 1) / P;
  };
  for (int pass = 0; pass < 2; ++pass) {
    // pass 0 counts units per size bucket, pass 1 writes them.  put() takes
    // a run of n partitions of one size with one atomic: record i of the
    // run is `r` with partition slot + i and token range shifted by i * P.
    auto put = [&](int size, const URec& r, int n) {
      if (n <= 0) return;
      const int b = bucket(size);
      if (pass == 0) {
        atomicAdd(&hist[b], n);
        return;
      }
      const int at = atomicAdd(&hist[b], n);
      if (n > 2) {                     // a longer run: queued for a whole wave
        const int li = atomicAdd(&s_nlong, 1);
        if (li < kPlanLongRuns) {
          s_lrec[li] = r;
          s_lat[li] = at;
          s_ln[li] = n;
          return;
        }
      }
      for (int i = 0; i < n; ++i) pa.urecs[at + i] = run_record(r, i);
    };
    for (int gi = tid; gi < NG; gi += kPlanThreads) {
      const int np = prompt_parts(gi);
      if (np == 0) continue;
      URec r;
      r.s = -(gi + 1);
      r.first = gstart[gi];
      r.cnt = gstart[gi + 1] - r.first;
      r.lp = glp[gi];
      r.ts = members[r.first];                   // any member: all share the prompt's blocks
      r.pf = 0;
      r.tb = 0;
      r.te = P;
      put(P, r, np - 1);
      // the last partition: the rest of the prompt plus absorbed own tokens
      r.pf = (np - 1) | kUnitTail;
      r.tb = (np - 1) * P;
      r.te = r.lp;
      put(r.lp - r.tb + gabs[gi], r, 1);
    }
    for (int s = tid; s < B; s += kPlanThreads) {
      const SeqLayout lay = seq_layout(s);
      const int own = lay.nparts - lay.np_pre;
      if (pass == 0 && lay.nparts > 1) pa.split[atomicAdd(&s_split, 1)] = make_int2(s, lay.nparts);
      URec r;
      r.s = s;
      r.first = r.cnt = r.lp = 0;
      r.ts = s;
      if (lay.nparts == 0) {                     // empty or out of contract: one empty unit
        r.pf = kUnitDirect | (lay.bad ? kUnitBad : 0);
        r.tb = r.te = 0;
        put(0, r, 1);
      }
      if (own > 0) {
        const int flags = lay.nparts == 1 ? kUnitDirect : 0;
#if PA_BALANCED_PARTS
        const int span = lay.len - lay.lp;
        const int S = own == 1 ? P : ((span + own - 1) / own + 15) & ~15;
#else
        const int S = P;
#endif
        r.pf = lay.np_pre | flags;
        r.tb = lay.lp;
        r.te = lay.lp + S;
        put(S, r, own - 1);                      // full parts
        r.pf = (lay.np_pre + own - 1) | flags;
        r.tb = lay.lp + (own - 1) * S;
        r.te = lay.len;
        put(lay.len - r.tb, r, 1);
      }
    }
    __syncthreads();
    if (pass == 1) {
      // The queued runs: one wave per run, lane i writing records i, i + 64,
      // ... (consecutive records: coalesced stores).
      const int nl = min(s_nlong, kPlanLongRuns);
      for (int li = tid >> 6; li < nl; li += kPlanThreads / 64)
        for (int i = tid & 63; i < s_ln[li]; i += 64)
          pa.urecs[s_lat[li] + i] = run_record(s_lrec[li], i);
    }
    if (pass == 0) {
      // bucket counts -> bucket starts; hist[256] = number of units
      block_exclusive_scan(hist, hist, 256, s_tot);
      __syncthreads();
      if (tid == 0) {
        pa.n_units[0] = hist[256];
        pa.n_units[1] = s_split;      // 0: the reduce launch has nothing to do
      }
      __syncthreads();
    }
  }
}

__global__ __launch_bounds__(kPlanThreads) void k_plan(const PArgs pa) { plan_body(pa); }

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// Partitions whose accumulators one reduce wave loads at once.
#ifndef PA_REDUCE_INFLIGHT
#define PA_REDUCE_INFLIGHT 8
#endif

// One wave per (sequence, head) of the sequences the plan listed as split
// merges their partitions: with M = max_p m_p,
//   out = sum_p 2^(m_p-M) acc_p / sum_p 2^(m_p-M) l_p.
// Lanes first read the (m, l) pairs of 64 partitions at a time, then every
// lane accumulates its head-dim elements over the partitions in order
// p = 0, 1, ..., taking each weight from the lane that computed it, with
// eight loads in flight.  All sums run in a fixed order, so reruns give
// identical bits (the order of the list does not matter).
template <int DT, int D>
__global__ __launch_bounds__(256) void k_reduce(const KArgs a) {
  constexpr int EPL = D / 64;          // head-dim elements per lane (1 or 2)
  constexpr int U = PA_REDUCE_INFLIGHT;   // partition loads in flight
  const int lane = threadIdx.x & 63;
  const int total = a.n_units[1] * a.num_heads;
  for (int it = blockIdx.x * 4 + (threadIdx.x >> 6); it < total; it += gridDim.x * 4) {
    const int2 sp = a.split[it / a.num_heads];   // (sequence, partitions)
    const int item = sp.x * a.num_heads + it % a.num_heads;
    const int np = sp.y;
    const float2* ml = a.ws_ml + (size_t)item * a.max_parts;
    const float* pacc = a.ws_acc + (size_t)item * a.max_parts * D + lane * EPL;

    float M = kEmptyMax;
    for (int p = lane; p < np; p += 64) M = fmaxf(M, ml[p].x);
    M = wave_max(M);
    float lsum = 0.f;
    for (int p = lane; p < np; p += 64) lsum += ml[p].y * fast_exp2(ml[p].x - M);
    const float inv = 1.f / wave_sum(lsum);

    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    for (int p0 = 0; p0 < np; p0 += 64) {
      const float wl = p0 + lane < np ? fast_exp2(ml[p0 + lane].x - M) : 0.f;
      const int cnt = min(64, np - p0);
      auto add = [&](int j, const float* v) {
        const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                                      __builtin_bit_cast(int, wl), j));
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = fmaf(w, v[e], acc[e]);
      };
      int j = 0;
      for (; j + U <= cnt; j += U) {
        float v[U][EPL];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float* src = pacc + (size_t)(p0 + j + u) * D;
          if constexpr (EPL == 2) {
            const float2 t = *reinterpret_cast<const float2*>(src);
            v[u][0] = t.x;
            v[u][1] = t.y;
          } else {
            v[u][0] = src[0];
          }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) add(j + u, v[u]);
      }
      for (; j < cnt; ++j) {
        float v[EPL];
        const float* src = pacc + (size_t)(p0 + j) * D;
#pragma unroll
        for (int e = 0; e < EPL; ++e) v[e] = src[e];
        add(j, v);
      }
    }
#pragma unroll
    for (int e = 0; e < EPL; ++e)
      store_elem<DT>(a.out, (size_t)item * D + lane * EPL + e, acc[e] * inv);
  }
}

struct CArgs {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int32_t* tables;   // nullptr: a contiguous cache [B][Hkv][max_len][d]
  const int32_t* lens;
  int num_seqs, num_kv_heads, row_chunks, row_bytes, bs_log2, max_blocks, num_blocks;
  int max_len;             // longest valid length (max_blocks << bs_log2 when paged)
};

// One thread per 16-byte chunk of a (sequence, KV head) row; copies K and V
// into row L-1 of the sequence: through its table, or in its contiguous
// region.
__device__ __forceinline__ void write_chunk(const CArgs& a, int idx) {
  if (idx >= a.num_seqs * a.num_kv_heads * a.row_chunks) return;
  const int c = idx % a.row_chunks;
  const int sg = idx / a.row_chunks;
  const int g = sg % a.num_kv_heads;
  const int s = sg / a.num_kv_heads;
  const int len = a.lens[s];
  if (len < 1 || len > a.max_len) return;
  const int pos = len - 1;
  size_t dst;
  if (a.tables == nullptr) {
    dst = ((size_t)sg * a.max_len + pos) * a.row_bytes + (size_t)c * 16;
  } else {
    const int phys = a.tables[(size_t)s * a.max_blocks + (pos >> a.bs_log2)];
    if ((unsigned)phys >= (unsigned)a.num_blocks) return;
    const size_t tile = (size_t)a.row_bytes << a.bs_log2;
    dst = ((size_t)phys * a.num_kv_heads + g) * tile +
          (size_t)(pos & ((1 << a.bs_log2) - 1)) * a.row_bytes + (size_t)c * 16;
  }
  const size_t src = (size_t)sg * a.row_bytes + (size_t)c * 16;
  *reinterpret_cast<uint4*>(a.k_pool + dst) = *reinterpret_cast<const uint4*>(a.k_new + src);
  *reinterpret_cast<uint4*>(a.v_pool + dst) = *reinterpret_cast<const uint4*>(a.v_new + src);
}

__global__ __launch_bounds__(256) void k_cache_write(const CArgs a) {
  write_chunk(a, blockIdx.x * 256 + threadIdx.x);
}

// The new token's write and the split-K plan in one launch, for a decode
// step that does both: workgroup 0 (dispatched first) plans, the others
// write kPlanThreads chunks each.  Neither reads what the other writes (the
// plan reads lengths and groups; the write reads lengths, tables and new
// rows), and the partition launch that follows reads both.
__global__ __launch_bounds__(kPlanThreads) void k_write_plan(const CArgs c, const PArgs p) {
  if (blockIdx.x == 0) plan_body(p);
  else write_chunk(c, (blockIdx.x - 1) * kPlanThreads + threadIdx.x);
}

struct BArgs {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const int32_t* pairs;   // [n][2] (source block, destination block)
  int num_pairs, num_blocks;
  size_t block_bytes;     // num_kv_heads * block_size * head_dim * elem, a multiple of 16
};

// Copy whole blocks of both pools (every KV head), e.g. the private copy a
// shared, partly filled block gets before a write.  Workgroup (pair, piece):
// 256 threads move 16-byte chunks of one block with streaming loads and
// stores, four chunks of K and four of V per thread per round, all loaded
// before any is stored.  Pairs naming a block outside the pool are skipped.
__global__ __launch_bounds__(256) void k_copy_blocks(const BArgs a) {
  const int pair = blockIdx.y;
  const int src = a.pairs[2 * pair], dst = a.pairs[2 * pair + 1];
  if ((unsigned)src >= (unsigned)a.num_blocks || (unsigned)dst >= (unsigned)a.num_blocks ||
      src == dst)
    return;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int U = 4;
  const size_t n16 = a.block_bytes / 16;
  const u32x4* ks = reinterpret_cast<const u32x4*>(a.k_pool + (size_t)src * a.block_bytes);
  const u32x4* vs = reinterpret_cast<const u32x4*>(a.v_pool + (size_t)src * a.block_bytes);
  u32x4* kd = reinterpret_cast<u32x4*>(a.k_pool + (size_t)dst * a.block_bytes);
  u32x4* vd = reinterpret_cast<u32x4*>(a.v_pool + (size_t)dst * a.block_bytes);
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x; i0 < n16; i0 += U * stride) {
    u32x4 k[U], v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = i0 + u * stride;
      if (i < n16) {
        k[u] = __builtin_nontemporal_load(ks + i);
        v[u] = __builtin_nontemporal_load(vs + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = i0 + u * stride;
      if (i < n16) {
        __builtin_nontemporal_store(k[u], kd + i);
        __builtin_nontemporal_store(v[u], vd + i);
      }
    }
  }
}

// Move whole blocks between a device pool and a pinned host pool through
// the host pool's device mapping: workgroup (pair, piece) copies 16-byte
// chunks of K and V of one block, four of each per thread per round, all
// loaded before any is stored.  Up to kSwapPairs pairs travel in the kernel
// arguments (checked on the host).
constexpr int kSwapPairs = 256;
struct SArgs {
  uint8_t* dst_k;
  uint8_t* dst_v;
  const uint8_t* src_k;
  const uint8_t* src_v;
  size_t block_bytes;     // a multiple of 16
  int num_pairs;
  int2 pairs[kSwapPairs]; // (source block, destination block)
};
__global__ __launch_bounds__(256) void k_swap_blocks(const SArgs a) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  constexpr int U = 4;
  const int2 pr = a.pairs[blockIdx.y];
  const size_t n16 = a.block_bytes / 16;
  const u32x4* ks = reinterpret_cast<const u32x4*>(a.src_k + (size_t)pr.x * a.block_bytes);
  const u32x4* vs = reinterpret_cast<const u32x4*>(a.src_v + (size_t)pr.x * a.block_bytes);
  u32x4* kd = reinterpret_cast<u32x4*>(a.dst_k + (size_t)pr.y * a.block_bytes);
  u32x4* vd = reinterpret_cast<u32x4*>(a.dst_v + (size_t)pr.y * a.block_bytes);
  const size_t stride = (size_t)gridDim.x * 256;
  for (size_t i0 = (size_t)blockIdx.x * 256 + threadIdx.x; i0 < n16; i0 += U * stride) {
    u32x4 k[U], v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = i0 + u * stride;
      if (i < n16) {
        k[u] = __builtin_nontemporal_load(ks + i);
        v[u] = __builtin_nontemporal_load(vs + i);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t i = i0 + u * stride;
      if (i < n16) {
        __builtin_nontemporal_store(k[u], kd + i);
        __builtin_nontemporal_store(v[u], vd + i);
      }
    }
  }
}

// Read probe: workgroup w streams tiles order[w], order[w + G], ... of
// `tile_bytes` bytes each (a multiple of 4096), four tiles in flight, with
// the same 16-byte non-temporal loads as the decode kernels; the XOR of
// what it read reaches memory only if it equals a value it never takes,
// which keeps the loads without writing anything.
__global__ __launch_bounds__(256) void k_read_probe(const uint8_t* buf, size_t tile_bytes,
                                                    const int32_t* order, int ntiles,
                                                    uint32_t* sink) {
  constexpr int U = 4;
  const size_t chunks = tile_bytes / 16;
  uint4 x = make_uint4(0, 0, 0, 0);
  for (int t0 = blockIdx.x; t0 < ntiles; t0 += U * gridDim.x) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = t0 + u * gridDim.x;
      const int tile = t < ntiles ? order[t] : order[t0];
      v[u] = ld16_stream(buf + (size_t)tile * tile_bytes + (threadIdx.x % chunks) * 16);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      x.x ^= v[u].x; x.y ^= v[u].y; x.z ^= v[u].z; x.w ^= v[u].w;
    }
    for (size_t c = threadIdx.x + 256; c < chunks; c += 256) {   // tiles over 4 KiB
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int t = t0 + u * gridDim.x;
        const int tile = t < ntiles ? order[t] : order[t0];
        const uint4 w = ld16_stream(buf + (size_t)tile * tile_bytes + c * 16);
        x.x ^= w.x; x.y ^= w.y; x.z ^= w.z; x.w ^= w.w;
      }
    }
  }
  if ((x.x ^ x.y ^ x.z ^ x.w) == 0x9e3779b9u && x.x == 0x7f4a7c15u) sink[0] = x.x;
}

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

Divisor set_divisor(int d) {
  const int l = ilog2(d);
  Divisor v;
  v.m = (uint32_t)((((uint64_t)1 << (31 + l)) + (uint64_t)d - 1) / (uint64_t)d);
  v.shift = 31 + l;
  return v;
}

// Launch a kernel that takes one argument struct and return the status of
// this launch alone (not an error some earlier runtime call left behind).
template <typename A>
hipError_t launch1(void (*kernel)(A), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                   const A& arg) {
  void* args[] = {const_cast<A*>(&arg)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, st);
}

template <typename A, typename B>
hipError_t launch2(void (*kernel)(A, B), dim3 grid, dim3 block, size_t lds, hipStream_t st,
                   const A& a, const B& b) {
  void* args[] = {const_cast<A*>(&a), const_cast<B*>(&b)};
  return hipLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, args, lds, st);
}

// Kernel arguments of the new-token write; chunks = 16-byte pieces of the
// new rows (one thread each).  False if the grid would not fit an int.
bool make_cargs(const CacheWriteParams& p, CArgs& ca, long long& chunks) {
  const int eb = p.dtype == kF32 ? 4 : 2;
  ca.k_pool = static_cast<uint8_t*>(p.k_pool);
  ca.v_pool = static_cast<uint8_t*>(p.v_pool);
  ca.k_new = static_cast<const uint8_t*>(p.k_new);
  ca.v_new = static_cast<const uint8_t*>(p.v_new);
  ca.tables = p.block_tables;
  ca.lens = p.context_lens;
  ca.num_seqs = p.num_seqs;
  ca.num_kv_heads = p.num_kv_heads;
  ca.row_bytes = p.head_dim * eb;
  ca.row_chunks = ca.row_bytes / 16;
  const bool contiguous = p.block_tables == nullptr;
  ca.bs_log2 = contiguous ? 0 : ilog2(p.block_size);
  ca.max_blocks = p.max_blocks_per_seq;
  ca.num_blocks = p.num_blocks;
  ca.max_len = contiguous ? p.max_len : p.max_blocks_per_seq * p.block_size;
  chunks = (long long)p.num_seqs * p.num_kv_heads * ca.row_chunks;
  return chunks <= 0x7fffffffLL - 1024;
}

constexpr size_t kOneWorkgroupPerCuLds = 81 * 1024;

template <int DT, int D, int W, int GW, bool PLAN>
hipError_t launch_decode_t(const KArgs& ka, int layout, bool nt, int grid, hipStream_t st) {
  const dim3 gd(grid), bd(W * 64);
  // Split-K partitions of 512 tokens or more run one 8-wave workgroup per CU
  // (measured faster than two on the long-context batch): the unused dynamic
  // LDS below is over half of a CU's 160 KiB, so a second one does not fit.
  const size_t lds = (W == 8 && PLAN) ? kOneWorkgroupPerCuLds : 0;
  // The new-token write inside a single pass (the host checks the case).
  if (ka.k_new != nullptr) {
    if constexpr (!PLAN && GW == 1) {
      if (layout == kBigPages && nt)
        return launch1(k_decode<DT, D, W, GW, kBigPages, true, false, true>, gd, bd, lds, st, ka);
    }
    return hipErrorInvalidValue;
  }
  // A contiguous cache holds no shared rows: streaming loads only.
  if (layout == kContiguous)
    return launch1(k_decode<DT, D, W, GW, kContiguous, true, PLAN>, gd, bd, lds, st, ka);
  if (layout == kBigPages) {
    if (nt) return launch1(k_decode<DT, D, W, GW, kBigPages, true, PLAN>, gd, bd, lds, st, ka);
    return launch1(k_decode<DT, D, W, GW, kBigPages, false, PLAN>, gd, bd, lds, st, ka);
  }
  if (nt) return launch1(k_decode<DT, D, W, GW, kSmallPages, true, PLAN>, gd, bd, lds, st, ka);
  return launch1(k_decode<DT, D, W, GW, kSmallPages, false, PLAN>, gd, bd, lds, st, ka);
}

// Waves per workgroup: a single pass uses 16 for one query head per wave
// and rows of at most 256 bytes (the two register buffers then fit in 128
// VGPRs), else 8; split-K uses 8 for partitions of 512 tokens or more, else 4.
template <int DT, int D>
hipError_t dispatch_gw(const KArgs& ka, int gw, int waves, int layout, bool nt, int grid,
                       hipStream_t st) {
  if (ka.urecs == nullptr) {
    switch (gw) {
      case 1:
        if constexpr (D * Elem<DT>::bytes <= 256)
          if (waves >= 16) return launch_decode_t<DT, D, 16, 1, false>(ka, layout, nt, grid, st);
        return launch_decode_t<DT, D, 8, 1, false>(ka, layout, nt, grid, st);
      case 2: return launch_decode_t<DT, D, 8, 2, false>(ka, layout, nt, grid, st);
      default: return launch_decode_t<DT, D, 8, 4, false>(ka, layout, nt, grid, st);
    }
  }
  switch (gw) {
    case 1:
      if (waves >= 8) return launch_decode_t<DT, D, 8, 1, true>(ka, layout, nt, grid, st);
      return launch_decode_t<DT, D, 4, 1, true>(ka, layout, nt, grid, st);
    case 2:
      if (waves >= 8) return launch_decode_t<DT, D, 8, 2, true>(ka, layout, nt, grid, st);
      return launch_decode_t<DT, D, 4, 2, true>(ka, layout, nt, grid, st);
    default:
      if (waves >= 8) return launch_decode_t<DT, D, 8, 4, true>(ka, layout, nt, grid, st);
      return launch_decode_t<DT, D, 4, 4, true>(ka, layout, nt, grid, st);
  }
}

template <int DT>
hipError_t dispatch_d(const KArgs& ka, int d, int gw, int waves, int layout, bool nt, int grid,
                      hipStream_t st) {
  return d == 64 ? dispatch_gw<DT, 64>(ka, gw, waves, layout, nt, grid, st)
                 : dispatch_gw<DT, 128>(ka, gw, waves, layout, nt, grid, st);
}

template <int DT, int D, int W>
hipError_t launch_mfma_t(const KArgs& ka, int layout, bool nt, int grid, size_t lds,
                         hipStream_t st) {
  const dim3 gd(grid), bd(W * 64);
  if (layout == kContiguous)
    return launch1(k_decode_mfma<DT, D, W, kContiguous, true>, gd, bd, lds, st, ka);
  if (layout == kBigPages) {
    if (nt) return launch1(k_decode_mfma<DT, D, W, kBigPages, true>, gd, bd, lds, st, ka);
    return launch1(k_decode_mfma<DT, D, W, kBigPages, false>, gd, bd, lds, st, ka);
  }
  if (nt) return launch1(k_decode_mfma<DT, D, W, kSmallPages, true>, gd, bd, lds, st, ka);
  return launch1(k_decode_mfma<DT, D, W, kSmallPages, false>, gd, bd, lds, st, ka);
}

// Waves per workgroup of the vector kernel for partitions of 512 tokens or
// more.
#ifndef PA_SPLIT_WAVES
#define PA_SPLIT_WAVES 8
#endif

// Bytes of consecutive head tiles of one block that an XCD reads as a group
// (xcd_group).
#ifndef PA_XCD_GROUP_BYTES
#define PA_XCD_GROUP_BYTES 8192
#endif

#ifndef PA_REDUCE_MAX_WGS
#define PA_REDUCE_MAX_WGS 1024
#endif

// Most workgroups a split-K partition launch starts (see launch_decode).
#ifndef PA_MAX_GRID_WGS
#define PA_MAX_GRID_WGS 4096
#endif

// Smallest query-head group sent to the matrix-core kernel.
#ifndef PA_MFMA_MIN_GROUP
#define PA_MFMA_MIN_GROUP 2
#endif

// Waves per workgroup of the matrix-core kernel.  Each wave holds two
// 16-token K/V slots in LDS (16 KiB at head_dim 128); two workgroups of four
// waves fill 128 KiB of the 160 KiB of LDS per CU.
#ifndef PA_MFMA_WAVES
#define PA_MFMA_WAVES 4
#endif

template <int DT>
hipError_t dispatch_mfma(const KArgs& ka, int d, int layout, bool nt, int grid, hipStream_t st) {
  constexpr int W = PA_MFMA_WAVES;
  // Two slots of one 16-token K tile and V tile per wave; the merge of the
  // waves after the loop reuses them.
  const size_t lds = (size_t)W * 2 * 2 * 16 * d * 2;
  if (d == 64) return launch_mfma_t<DT, 64, W>(ka, layout, nt, grid, lds, st);
  return launch_mfma_t<DT, 128, W>(ka, layout, nt, grid, lds, st);
}

template <int DT>
hipError_t launch_reduce_t(const KArgs& ka, int d, int grid, hipStream_t st) {
  if (d == 64) return launch1(k_reduce<DT, 64>, dim3(grid), dim3(256), 0, st, ka);
  return launch1(k_reduce<DT, 128>, dim3(grid), dim3(256), 0, st, ka);
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  const bool shared = p.seq_group != nullptr;
  KArgs ka;
  ka.out = p.out;
  ka.q = static_cast<const uint8_t*>(p.q);
  ka.k_pool = static_cast<const uint8_t*>(p.k_pool);
  ka.v_pool = static_cast<const uint8_t*>(p.v_pool);
  ka.tables = p.block_tables;
  ka.lens = p.context_lens;
  ka.k_new = nullptr;
  ka.v_new = nullptr;
  uint8_t* ws = reinterpret_cast<uint8_t*>(p.workspace);
  const WsLayout wl = ws_layout(p.num_seqs, p.num_heads, p.head_dim, p.max_partitions,
                                shared ? p.num_groups : -1);
  ka.ws_acc = p.workspace;
  ka.ws_ml = ws ? reinterpret_cast<float2*>(ws + wl.ml) : nullptr;
  ka.n_units = ws ? reinterpret_cast<const int*>(ws + wl.n_units) : nullptr;
  ka.urecs = ws ? reinterpret_cast<const URec*>(ws + wl.units) : nullptr;
  ka.split = ws ? reinterpret_cast<const int2*>(ws + wl.split) : nullptr;
  ka.minfo = shared ? reinterpret_cast<const int4*>(ws + wl.minfo) : nullptr;
  // The caller's groups: read by the plan only.
  ka.seq_group = shared ? p.seq_group : nullptr;
  ka.group_prefix = shared ? p.group_prefix : nullptr;
  ka.num_groups = shared ? p.num_groups : 0;
  ka.max_units = (int)wl.max_units;
  ka.num_seqs = p.num_seqs;
  ka.num_heads = p.num_heads;
  ka.num_kv_heads = p.num_kv_heads;
  const bool contiguous = p.block_tables == nullptr;
  // A contiguous cache is described to the kernels as one block of max_len
  // rows per sequence, block s for sequence s.
  ka.bs_log2 = contiguous ? 0 : ilog2(p.block_size);
  ka.max_blocks = p.max_blocks_per_seq;
  ka.num_blocks = contiguous ? p.num_seqs : p.num_blocks;
  ka.max_len = contiguous ? p.max_len : p.max_blocks_per_seq * p.block_size;
  ka.group = p.num_heads / p.num_kv_heads;
  // Grouped heads in 16-bit types run on the matrix cores (chunks of up to 16
  // query columns per workgroup); fp32, single heads, or the VALU-only flag
  // use the vector path (chunks of GW heads).  Shared-prompt decode always
  // runs on the matrix cores: a prompt unit's columns are the queries of all
  // members of a group.
  const bool mfma = shared || (p.dtype != kF32 && ka.group >= PA_MFMA_MIN_GROUP &&
                               !(p.flags & kFlagValuOnly));
  const int gw = ka.group % 4 == 0 ? 4 : (ka.group % 2 == 0 ? 2 : 1);
  const int cols = shared ? ka.group * (p.max_group_size > 1 ? p.max_group_size : 1) : ka.group;
  ka.chunks = mfma ? (cols + 15) / 16 : ka.group / gw;
  ka.part_tokens = p.partition_size;
  ka.part_div = set_divisor(std::max(1, p.partition_size));
  ka.members_chunk = 16 % ka.group == 0 ? 16 / ka.group : 16 / ka.group + 2;
  ka.max_parts = p.max_partitions;
  ka.scale_log2 = p.scale * kLog2e;
  // Streaming (non-temporal) K/V loads unless blocks are shared.
  const bool nt = !(p.flags & kFlagSharedKV);
  const int layout = contiguous ? kContiguous : p.block_size >= 16 ? kBigPages : kSmallPages;
  // A single pass gives each workgroup a whole sequence: many waves shorten
  // its critical path and let the dispatcher balance ragged lengths.  A
  // partition of P tokens has P/16 steps; keep at least four per wave.
  int waves;
  const int row_bytes = p.head_dim * (p.dtype == kF32 ? 4 : 2);
  if (p.workspace == nullptr) waves = gw == 1 && row_bytes <= 256 ? PA_VALU_SINGLE_WAVES : 8;
  else waves = p.partition_size >= 512 ? PA_SPLIT_WAVES : 4;
  // One pass of the grid covers grid_units units: every sequence without a
  // plan; with one, the unit list's capacity, capped at PA_MAX_GRID_WGS
  // workgroups (the workgroups then take further units in snake order), so
  // that few workgroups find no unit when the plan lists far fewer units
  // than the capacity bound.
  const long long H = (long long)ka.chunks * p.num_kv_heads;
  long long units = p.num_seqs;
  if (ws != nullptr) {
    units = (long long)wl.max_units;
    units = std::min(units, std::max(1LL, (long long)PA_MAX_GRID_WGS / H));
  }
  ka.grid_units = (int)units;
  const long long grid = H * units;
  if (grid <= 0 || grid > 0x7fffffffLL || wl.max_units > 0x7fffffffULL)
    return hipErrorInvalidConfiguration;
  // Heads per XCD group: the largest power of two c with c tiles of one
  // (block, KV head) within PA_XCD_GROUP_BYTES, c dividing the workgroups of
  // a unit and 8c dividing the grid (so the renumbering is a bijection).
  {
    const long long tile = (long long)p.head_dim * (p.dtype == kF32 ? 4 : 2) *
                           (contiguous ? p.max_len : p.block_size);
    const int H = ka.chunks * p.num_kv_heads;
    int c = 1;
    while (2LL * c * tile <= PA_XCD_GROUP_BYTES && H % (2 * c) == 0 && grid % (16LL * c) == 0)
      c *= 2;
    ka.xcd_heads = c;
  }

  hipError_t e;
  if (ws != nullptr) {
    PArgs pa_;
    pa_.k = ka;
    pa_.n_units = reinterpret_cast<int*>(ws + wl.n_units);
    pa_.urecs = reinterpret_cast<URec*>(ws + wl.units);
    pa_.split = reinterpret_cast<int2*>(ws + wl.split);
    pa_.minfo = shared ? reinterpret_cast<int4*>(ws + wl.minfo) : nullptr;
    pa_.arrival = shared ? reinterpret_cast<int*>(ws + wl.arrival) : nullptr;
    pa_.group_fill = shared ? reinterpret_cast<int*>(ws + wl.group_fill) : nullptr;
    pa_.group_start = shared ? reinterpret_cast<int*>(ws + wl.group_start) : nullptr;
    pa_.group_lp = shared ? reinterpret_cast<int*>(ws + wl.group_lp) : nullptr;
    pa_.max_group_size = p.max_group_size;
    if (p.write != nullptr) {
      // The new token's write rides in the plan's launch (workgroups 1..).
      CArgs ca;
      long long chunks;
      if (!make_cargs(*p.write, ca, chunks)) return hipErrorInvalidConfiguration;
      const int wgs = 1 + (int)((chunks + kPlanThreads - 1) / kPlanThreads);
      e = launch2(k_write_plan, dim3(wgs), dim3(kPlanThreads), 0, stream, ca, pa_);
    } else {
      e = launch1(k_plan, dim3(1), dim3(kPlanThreads), 0, stream, pa_);
    }
    if (e != hipSuccess) return e;
  } else if (p.write != nullptr) {
    // A single pass of the vector kernel over blocks of 16 tokens or more
    // writes the new token itself (k_decode's FUSED); otherwise the write
    // is its own launch before the decode.
    if (!mfma && gw == 1 && layout == kBigPages && nt) {
      ka.k_new = static_cast<const uint8_t*>(p.write->k_new);
      ka.v_new = static_cast<const uint8_t*>(p.write->v_new);
    } else {
      e = launch_cache_write(*p.write, stream);
      if (e != hipSuccess) return e;
    }
  }
  if (mfma) {
    e = p.dtype == kF16 ? dispatch_mfma<kF16>(ka, p.head_dim, layout, nt, (int)grid, stream)
                        : dispatch_mfma<kBF16>(ka, p.head_dim, layout, nt, (int)grid, stream);
  } else {
    switch (p.dtype) {
      case kF32: e = dispatch_d<kF32>(ka, p.head_dim, gw, waves, layout, nt, (int)grid, stream); break;
      case kF16: e = dispatch_d<kF16>(ka, p.head_dim, gw, waves, layout, nt, (int)grid, stream); break;
      default: e = dispatch_d<kBF16>(ka, p.head_dim, gw, waves, layout, nt, (int)grid, stream); break;
    }
  }
  if (e != hipSuccess || ws == nullptr) return e;
  // One wave per (split sequence, head), at most PA_REDUCE_MAX_WGS
  // workgroups of four waves striding over them (the count is on the device).
  const int rgrid = std::min((p.num_seqs * p.num_heads + 3) / 4, PA_REDUCE_MAX_WGS);
  switch (p.dtype) {
    case kF32: return launch_reduce_t<kF32>(ka, p.head_dim, rgrid, stream);
    case kF16: return launch_reduce_t<kF16>(ka, p.head_dim, rgrid, stream);
    default: return launch_reduce_t<kBF16>(ka, p.head_dim, rgrid, stream);
  }
}

// Scratch for callers that cannot allocate device memory: the split-K
// workspace of the no-allocation decode entry lives in this file-scope array.
// Every GPU the library runs on holds its own copy, at its own address, until
// the process ends; every call on one GPU uses that GPU's copy, so calls that
// overlap on one GPU race.  In host code the array's name is only a stand-in
// for the symbol: kernels and copies get the device address that
// noalloc_scratch() looked up for the current device.
static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_copy_blocks(void* k_pool, void* v_pool, const int32_t* pairs, int num_pairs,
                              int num_blocks, size_t block_bytes, hipStream_t stream) {
  if (num_pairs == 0) return hipSuccess;
  BArgs a;
  a.k_pool = static_cast<uint8_t*>(k_pool);
  a.v_pool = static_cast<uint8_t*>(v_pool);
  a.pairs = pairs;
  a.num_pairs = num_pairs;
  a.num_blocks = num_blocks;
  a.block_bytes = block_bytes;
  const size_t chunks = block_bytes / 16;
  const int pieces = (int)std::min<size_t>((chunks + 1023) / 1024, 64);   // 4 chunks per thread
  // (each thread of a piece then copies one round of four chunks of K and V)
  return launch1(k_copy_blocks, dim3(pieces, num_pairs), dim3(256), 0, stream, a);
}

hipError_t launch_swap_blocks(void* dst_k, void* dst_v, const void* src_k, const void* src_v,
                              const int32_t* pairs, int num_pairs, size_t block_bytes,
                              hipStream_t stream) {
  SArgs a;
  a.dst_k = static_cast<uint8_t*>(dst_k);
  a.dst_v = static_cast<uint8_t*>(dst_v);
  a.src_k = static_cast<const uint8_t*>(src_k);
  a.src_v = static_cast<const uint8_t*>(src_v);
  a.block_bytes = block_bytes;
  const size_t chunks = block_bytes / 16;
  const int pieces = (int)std::min<size_t>((chunks + 1023) / 1024, 64);
  for (int first = 0; first < num_pairs; first += kSwapPairs) {
    a.num_pairs = std::min(kSwapPairs, num_pairs - first);
    for (int i = 0; i < a.num_pairs; ++i)
      a.pairs[i] = make_int2(pairs[2 * (first + i)], pairs[2 * (first + i) + 1]);
    const hipError_t e = launch1(k_swap_blocks, dim3(pieces, a.num_pairs), dim3(256), 0, stream, a);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_read_probe(const void* buf, size_t tile_bytes, const int32_t* order,
                             int ntiles, uint32_t* sink, hipStream_t stream) {
  if (ntiles == 0) return hipSuccess;
  const int grid = std::min(ntiles, 4096);
  const uint8_t* b = static_cast<const uint8_t*>(buf);
  void* args[] = {&b, &tile_bytes, &order, &ntiles, &sink};
  return hipLaunchKernel(reinterpret_cast<const void*>(k_read_probe), dim3(grid), dim3(256), args,
                         0, stream);
}

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  CArgs ca;
  long long total;
  if (!make_cargs(p, ca, total)) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 255) / 256);
  return launch1(k_cache_write, dim3(grid), dim3(256), 0, stream, ca);
}

}  // namespace pa
