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

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Partition bookkeeping shared by the partition and reduce kernels.  A length
// outside [0, max_blocks*bs], or needing more partitions than the grid holds,
// is a contract violation: the sequence is flagged and its output set to NaN.
struct SeqParts {
  int len;
  int nparts;     // ceil(len / P); 0 for an empty sequence
  bool bad;
};
__device__ __forceinline__ SeqParts seq_parts(int len, int P, int max_parts, int max_blocks,
                                              int bs_log2) {
  SeqParts r;
  r.bad = len < 0 || len > (max_blocks << bs_log2);
  r.len = r.bad ? 0 : len;
  r.nparts = (r.len + P - 1) / P;
  if (r.nparts > max_parts) r.bad = true;
  if (r.bad) { r.len = 0; r.nparts = 0; }
  return r;
}

struct KArgs {
  void* out;
  const uint8_t* q;
  const uint8_t* k_pool;
  const uint8_t* v_pool;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_acc;        // [B][Hq][max_parts][D]
  float2* ws_ml;        // [B][Hq][max_parts] of (max, sum)
  int num_seqs, num_heads, num_kv_heads, bs_log2, max_blocks, num_blocks;
  int group;            // query heads per KV head
  int chunks;           // group / GW
  int part_tokens;      // P
  int max_parts;
  float scale_log2;     // scale * log2(e)
  int streaming;        // nonzero: K/V loads carry the non-temporal hint
};

// One workgroup = (sequence s, KV head g, chunk of GW query heads, partition p).
// Its W waves take the partition's 16-token steps round-robin.
template <int DT, int D, int W, int GW, bool BIG_BLOCKS>
__global__ __launch_bounds__(W * 64) void k_decode(const KArgs a) {
  constexpr int EB = Elem<DT>::bytes;
  constexpr int ROWB = D * EB;           // bytes per token row of one head
  constexpr int LPR = ROWB / 16;         // lanes per row
  constexpr int RPL = 64 / LPR;          // rows per wave-wide load
  constexpr int NL = 16 / RPL;           // loads per 16-token step
  constexpr int EPL = 16 / EB;           // elements per lane slice
  static_assert(LPR >= 4 && LPR <= 32 && RPL * LPR == 64 && NL * RPL == 16, "row shape");

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int r = lane / LPR;              // row group
  const int c = lane % LPR;              // 16-byte slice within the row

  int wg = blockIdx.x;
  const int ch = wg % a.chunks;  wg /= a.chunks;
  const int g = wg % a.num_kv_heads;  wg /= a.num_kv_heads;
  const int s = wg % a.num_seqs;
  const int p = wg / a.num_seqs;

  const SeqParts sp = seq_parts(a.lens[s], a.part_tokens, a.max_parts, a.max_blocks, a.bs_log2);
  const bool direct = sp.nparts <= 1;    // the only partition writes the output itself
  if (p >= (sp.nparts > 1 ? sp.nparts : 1)) return;
  const int t_begin = p * a.part_tokens;
  const int t_end = min(t_begin + a.part_tokens, sp.len);
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

  const int bs_mask = (1 << a.bs_log2) - 1;
  const size_t tile_bytes = (size_t)ROWB << a.bs_log2;          // one (block, head) tile
  const size_t block_bytes = tile_bytes * a.num_kv_heads;
  const int32_t* trow = a.tables + (size_t)s * a.max_blocks;
  bool bad_block = false;

  // Iteration k of this wave handles the 16-token step starting at step_t0(k).
  const int nk = nsteps > wave ? (nsteps - wave + W - 1) / W : 0;
  auto step_t0 = [&](int k) { return t_begin + ((wave + k * W) << 4); };
  // block_size >= 16: a step lies in one block, whose id is read once per step
  // (a wave-uniform scalar load, issued two steps ahead of its use).
  auto step_phys = [&](int k) -> int {
    if constexpr (BIG_BLOCKS) return trow[step_t0(k) >> a.bs_log2];
    else return 0;
  };
  auto load_step_t = [&](auto nt, int k, int phys, uint4 (&kr)[NL], uint4 (&vr)[NL]) {
    constexpr bool NT = decltype(nt)::value;
    const int t0 = step_t0(k);
    if constexpr (BIG_BLOCKS) {
      if ((unsigned)phys >= (unsigned)a.num_blocks) { bad_block = true; phys = 0; }
      const size_t tile = (size_t)phys * block_bytes + (size_t)g * tile_bytes;
      const uint8_t* kb = a.k_pool + tile + (size_t)(t0 & bs_mask) * ROWB + c * 16;
      const uint8_t* vb = a.v_pool + tile + (size_t)(t0 & bs_mask) * ROWB + c * 16;
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int dt = min(i * RPL + r, t_end - 1 - t0);   // last valid row past the end
        kr[i] = ld16<NT>(kb + dt * ROWB);
      }
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int dt = min(i * RPL + r, t_end - 1 - t0);
        vr[i] = ld16<NT>(vb + dt * ROWB);
      }
    } else {
      // block_size < 16: each row looks up its own block.
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int t = min(t0 + i * RPL + r, t_end - 1);
        int ph = trow[t >> a.bs_log2];
        if ((unsigned)ph >= (unsigned)a.num_blocks) { bad_block = true; ph = 0; }
        const size_t off = (size_t)ph * block_bytes + (size_t)g * tile_bytes +
                           (size_t)(t & bs_mask) * ROWB + c * 16;
        kr[i] = ld16<NT>(a.k_pool + off);
        vr[i] = ld16<NT>(a.v_pool + off);
      }
    }
  };
  auto load_step = [&](int k, int phys, uint4 (&kr)[NL], uint4 (&vr)[NL]) {
    if (a.streaming) load_step_t(std::true_type{}, k, phys, kr, vr);
    else load_step_t(std::false_type{}, k, phys, kr, vr);
  };
  auto compute_step = [&](int k, const uint4 (&kr)[NL], const uint4 (&vr)[NL]) {
    const int t0 = step_t0(k);
    float sc[GW][NL];
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const bool valid = t0 + i * RPL + r < t_end;
#pragma unroll
      for (int hh = 0; hh < GW; ++hh) {
        const float z = row_group_sum<LPR>(dot16<DT>(kr[i], qv[hh], 0.f)) * a.scale_log2;
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
      for (int hh = 0; hh < GW; ++hh) Axpy<DT>::run(acc[hh], sc[hh][i], vr[i]);
  };

  // Two register buffers: the loads of step k+1 are in flight while step k
  // is computed.
  uint4 kA[NL], vA[NL], kB[NL], vB[NL];
  int physA = 0, physB = 0;
  if (nk > 0) { physA = step_phys(0); load_step(0, physA, kA, vA); }
  if (nk > 1) physB = step_phys(1);
  for (int k = 0; k < nk; k += 2) {
    if (k + 1 < nk) load_step(k + 1, physB, kB, vB);
    if (k + 2 < nk) physA = step_phys(k + 2);
    compute_step(k, kA, vA);
    if (k + 1 >= nk) break;
    if (k + 2 < nk) load_step(k + 2, physA, kA, vA);
    if (k + 3 < nk) physB = step_phys(k + 3);
    compute_step(k + 1, kB, vB);
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
      for (int e = 0; e < EPL; ++e) acc[hh][e] = acc[hh][e] * fa + __shfl_xor(acc[hh][e], off) * fb;
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
  const bool poisoned = sp.bad || s_bad;
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
}

struct RArgs {
  void* out;
  const int32_t* lens;
  const float* ws_acc;
  const float2* ws_ml;
  int num_seqs, num_heads, max_blocks, bs_log2;
  int part_tokens, max_parts;
};

// One wave per (sequence, head): merge the partitions in order p = 0, 1, ...
template <int DT, int D>
__global__ __launch_bounds__(256) void k_reduce(const RArgs a) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= a.num_seqs * a.num_heads) return;
  const int s = item / a.num_heads;
  const SeqParts sp = seq_parts(a.lens[s], a.part_tokens, a.max_parts, a.max_blocks, a.bs_log2);
  if (sp.bad || sp.nparts <= 1) return;   // written by the partition kernel
  const float2* ml = a.ws_ml + (size_t)item * a.max_parts;
  const float* pacc = a.ws_acc + (size_t)item * a.max_parts * D;
  float M = kEmptyMax;
  for (int p = 0; p < sp.nparts; ++p) M = fmaxf(M, ml[p].x);
  float lsum = 0.f;
  for (int p = 0; p < sp.nparts; ++p) lsum += ml[p].y * fast_exp2(ml[p].x - M);
  const float inv = 1.f / lsum;
  for (int e = lane; e < D; e += 64) {
    float asum = 0.f;
    for (int p = 0; p < sp.nparts; ++p) asum += pacc[(size_t)p * D + e] * fast_exp2(ml[p].x - M);
    store_elem<DT>(a.out, (size_t)item * D + e, asum * inv);
  }
}

struct CArgs {
  uint8_t* k_pool;
  uint8_t* v_pool;
  const uint8_t* k_new;
  const uint8_t* v_new;
  const int32_t* tables;
  const int32_t* lens;
  int num_seqs, num_kv_heads, row_chunks, row_bytes, bs_log2, max_blocks, num_blocks;
};

// One thread per 16-byte chunk of a (sequence, KV head) row; copies K and V.
__global__ __launch_bounds__(256) void k_cache_write(const CArgs a) {
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= a.num_seqs * a.num_kv_heads * a.row_chunks) return;
  const int c = idx % a.row_chunks;
  const int sg = idx / a.row_chunks;
  const int g = sg % a.num_kv_heads;
  const int s = sg / a.num_kv_heads;
  const int len = a.lens[s];
  if (len < 1 || len > (a.max_blocks << a.bs_log2)) return;
  const int pos = len - 1;
  const int phys = a.tables[(size_t)s * a.max_blocks + (pos >> a.bs_log2)];
  if ((unsigned)phys >= (unsigned)a.num_blocks) return;
  const size_t tile = (size_t)a.row_bytes << a.bs_log2;
  const size_t dst = ((size_t)phys * a.num_kv_heads + g) * tile +
                     (size_t)(pos & ((1 << a.bs_log2) - 1)) * a.row_bytes + (size_t)c * 16;
  const size_t src = (size_t)sg * a.row_bytes + (size_t)c * 16;
  *reinterpret_cast<uint4*>(a.k_pool + dst) = *reinterpret_cast<const uint4*>(a.k_new + src);
  *reinterpret_cast<uint4*>(a.v_pool + dst) = *reinterpret_cast<const uint4*>(a.v_new + src);
}

int ilog2(int x) {
  int r = 0;
  while ((1 << r) < x) ++r;
  return r;
}

template <int DT, int D, int W, int GW>
hipError_t launch_decode_t(const KArgs& ka, bool big, int grid, hipStream_t st) {
  if (big) hipLaunchKernelGGL((k_decode<DT, D, W, GW, true>), dim3(grid), dim3(W * 64), 0, st, ka);
  else hipLaunchKernelGGL((k_decode<DT, D, W, GW, false>), dim3(grid), dim3(W * 64), 0, st, ka);
  return hipGetLastError();
}

// Waves per workgroup: 16 only for one query head per wave and rows of at
// most 256 bytes (the two register buffers then fit in 128 VGPRs), else 8 or 4.
template <int DT, int D>
hipError_t dispatch_gw(const KArgs& ka, int gw, int waves, bool big, int grid, hipStream_t st) {
  switch (gw) {
    case 1:
      if constexpr (D * Elem<DT>::bytes <= 256)
        if (waves >= 16) return launch_decode_t<DT, D, 16, 1>(ka, big, grid, st);
      if (waves >= 8) return launch_decode_t<DT, D, 8, 1>(ka, big, grid, st);
      return launch_decode_t<DT, D, 4, 1>(ka, big, grid, st);
    case 2:
      if (waves >= 8) return launch_decode_t<DT, D, 8, 2>(ka, big, grid, st);
      return launch_decode_t<DT, D, 4, 2>(ka, big, grid, st);
    default:
      if (waves >= 8) return launch_decode_t<DT, D, 8, 4>(ka, big, grid, st);
      return launch_decode_t<DT, D, 4, 4>(ka, big, grid, st);
  }
}

template <int DT>
hipError_t dispatch_d(const KArgs& ka, int d, int gw, int waves, bool big, int grid,
                      hipStream_t st) {
  return d == 64 ? dispatch_gw<DT, 64>(ka, gw, waves, big, grid, st)
                 : dispatch_gw<DT, 128>(ka, gw, waves, big, grid, st);
}

template <int DT>
hipError_t launch_reduce_t(const RArgs& ra, int d, int grid, hipStream_t st) {
  if (d == 64) hipLaunchKernelGGL((k_reduce<DT, 64>), dim3(grid), dim3(256), 0, st, ra);
  else hipLaunchKernelGGL((k_reduce<DT, 128>), dim3(grid), dim3(256), 0, st, ra);
  return hipGetLastError();
}

}  // namespace

size_t splitk_partial_bytes(int num_seqs, int num_heads, int head_dim, int max_partitions) {
  const size_t slots = (size_t)num_seqs * num_heads * max_partitions;
  return slots * head_dim * sizeof(float) + slots * sizeof(float2);
}

hipError_t launch_decode(const DecodeParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  KArgs ka;
  ka.out = p.out;
  ka.q = static_cast<const uint8_t*>(p.q);
  ka.k_pool = static_cast<const uint8_t*>(p.k_pool);
  ka.v_pool = static_cast<const uint8_t*>(p.v_pool);
  ka.tables = p.block_tables;
  ka.lens = p.context_lens;
  const size_t slots = (size_t)p.num_seqs * p.num_heads * p.max_partitions;
  ka.ws_acc = p.workspace;
  ka.ws_ml = p.workspace ? reinterpret_cast<float2*>(p.workspace + slots * p.head_dim) : nullptr;
  ka.num_seqs = p.num_seqs;
  ka.num_heads = p.num_heads;
  ka.num_kv_heads = p.num_kv_heads;
  ka.bs_log2 = ilog2(p.block_size);
  ka.max_blocks = p.max_blocks_per_seq;
  ka.num_blocks = p.num_blocks;
  ka.group = p.num_heads / p.num_kv_heads;
  const int gw = ka.group % 4 == 0 ? 4 : (ka.group % 2 == 0 ? 2 : 1);
  ka.chunks = ka.group / gw;
  ka.part_tokens = p.partition_size;
  ka.max_parts = p.max_partitions;
  ka.scale_log2 = p.scale * kLog2e;
  ka.streaming = (p.flags & kFlagSharedKV) ? 0 : 1;
  const bool big = p.block_size >= 16;
  // A single pass gives each workgroup a whole sequence: many waves shorten
  // its critical path and let the dispatcher balance ragged lengths.  A
  // partition of P tokens has P/16 steps; keep at least four per wave.
  int waves;
  const int row_bytes = p.head_dim * (p.dtype == kF32 ? 4 : 2);
  if (p.workspace == nullptr) waves = gw == 1 && row_bytes <= 256 ? 16 : 8;
  else waves = p.partition_size >= 512 ? 8 : 4;
  const long long grid = (long long)ka.chunks * p.num_kv_heads * p.num_seqs * p.max_partitions;
  if (grid <= 0 || grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;

  hipError_t e;
  switch (p.dtype) {
    case kF32: e = dispatch_d<kF32>(ka, p.head_dim, gw, waves, big, (int)grid, stream); break;
    case kF16: e = dispatch_d<kF16>(ka, p.head_dim, gw, waves, big, (int)grid, stream); break;
    default: e = dispatch_d<kBF16>(ka, p.head_dim, gw, waves, big, (int)grid, stream); break;
  }
  if (e != hipSuccess || p.workspace == nullptr) return e;

  RArgs ra;
  ra.out = p.out;
  ra.lens = p.context_lens;
  ra.ws_acc = ka.ws_acc;
  ra.ws_ml = ka.ws_ml;
  ra.num_seqs = p.num_seqs;
  ra.num_heads = p.num_heads;
  ra.max_blocks = p.max_blocks_per_seq;
  ra.bs_log2 = ka.bs_log2;
  ra.part_tokens = p.partition_size;
  ra.max_parts = p.max_partitions;
  const int rgrid = (p.num_seqs * p.num_heads + 3) / 4;
  switch (p.dtype) {
    case kF32: return launch_reduce_t<kF32>(ra, p.head_dim, rgrid, stream);
    case kF16: return launch_reduce_t<kF16>(ra, p.head_dim, rgrid, stream);
    default: return launch_reduce_t<kBF16>(ra, p.head_dim, rgrid, stream);
  }
}

hipError_t launch_cache_write(const CacheWriteParams& p, hipStream_t stream) {
  if (p.num_seqs == 0) return hipSuccess;
  const int eb = p.dtype == kF32 ? 4 : 2;
  CArgs ca;
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
  ca.bs_log2 = ilog2(p.block_size);
  ca.max_blocks = p.max_blocks_per_seq;
  ca.num_blocks = p.num_blocks;
  const long long total = (long long)p.num_seqs * p.num_kv_heads * ca.row_chunks;
  if (total > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const int grid = (int)((total + 255) / 256);
  hipLaunchKernelGGL(k_cache_write, dim3(grid), dim3(256), 0, stream, ca);
  return hipGetLastError();
}

}  // namespace pa
