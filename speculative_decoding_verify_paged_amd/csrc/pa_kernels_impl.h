// pa_kernels_impl.h — gfx950 kernels of paged verify attention (device code
// shared by the per-dtype translation units pa_segment_*.hip and pa_combine.hip).
//
// Two kernels per call:
//   1. pa_segment: one workgroup per (KV segment j, KV head, sequence) — for
//      a small batch (2..256 sequences, no more than the workgroup slots per
//      KV head), per (work-list chunk, KV head), a chunk being a run of one
//      sequence's steps whose size the device picks from the lengths so the
//      chunks fill one round of workgroups.  Its wavefronts stream the
//      segment's K/V page tiles straight from HBM into MFMA operand
//      registers, each tile read once for all G*T stacked query rows of the
//      GQA group, and keep an online softmax.  The workgroup merges its
//      wavefronts in LDS and writes one partial (O, m, l) per query row to
//      the workspace, indexed per token — or, with one segment, the
//      normalised output row itself.
//   2. pa_combine: log-sum-exp merge of the segment partials of each
//      (token, q head) row, cast to the output dtype (pa_finish instead for
//      one segment: only the check of subsequence_begins).
//
// Why segments: a verify call at batch 1 has only num_kv_heads independent
// KV streams; a kernel that gives each one workgroup idles almost all of the
// GPU (vLLM article "speculative decoding net loss": the use_3d gate passage,
// 128 workgroups falling to 8; OpenVINO issue #38153, "Performance issue
// description": the unpartitioned MIXED scan).  Splitting the key axis into
// segments reduced in parallel restores the parallelism, and the extra query
// rows ride along in the same MFMA tile (same article, direct kernel sweep:
// one extra row costs a fraction of a percent).
//
// Page layout.  A (block, KV head) page is a sequence of 16-slot sub-tiles,
// each stored in the register order of the MFMA operands that consume it, so
// that every wavefront load instruction (64 lanes x 16 B) reads 1 KB of
// contiguous memory — whole cache lines, which is what lets the loads keep
// enough requests in flight to approach the HBM streaming rate:
//   K: [d/32][(d%32)/8][slot%16][d%8]          (u8: [d/64][(d%64)/16][slot%16][d%16])
//   V: [d/32][(slot%16)/4][d%16][(d%32)/16][slot%4]
//                                               (u8: [d/64][(slot%16)/4][d%16][(d%64)/16][slot%4])
// Pages of 1, 2, 4 or 8 slots hold K row-major [slot][d] and V d-major
// [d][slot]; each lane gathers its own operand pieces from them.  With
// page_layout = kPagesRowMajor every page is [slot][d] for K and V; the
// wavefronts read whole page rows and reorder them into operand order
// through LDS.
//
// Data path of one wavefront step (32 keys = two sub-tiles, stacked rows
// r = g*T + i padded to 16):
//   S^T[slot, r] = K[slot, :] . Q[r, :]    v_mfma_f32_16x16x32, A = one K load per 32 d,
//                                           B = Q rows held in registers
//   online softmax per row (lane-local, two cross-lane max steps)
//   O^T[d, r] += V^T[d, key] . P^T[key, r]  v_mfma_f32_16x16x32 over all 32 keys,
//                                           A = half of each sub-tile's V load,
//                                           B = the S^T accumulators after exp
//                                           (bf16: hi + lo parts)
// The half-step path takes one sub-tile (16 keys) at a time, PV as
// v_mfma_f32_16x16x16 over its keys.  Every lane owns one stacked row
// r = lane % 16 in all three products, so the softmax state and its rescale
// never leave the lane.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pa_kernels.h"

namespace pav {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Launch a kernel that takes one argument struct; returns this launch's own
// error (not an earlier call's, as a later hipGetLastError would).  With
// events, the dispatch itself timestamps the kernel's start and end.
template <typename Args>
inline hipError_t launch_kernel(const void* fn, dim3 grid, dim3 block, hipStream_t st,
                                const Args& a, hipEvent_t ev0 = nullptr,
                                hipEvent_t ev1 = nullptr) {
  void* args[] = {const_cast<Args*>(&a)};
  if (ev0 || ev1) return hipExtLaunchKernel(fn, grid, block, args, 0, st, ev0, ev1, 0);
  return hipLaunchKernel(fn, grid, block, args, 0, st);
}

__device__ __forceinline__ u32x4 ld16(const char* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

// KV pages are read exactly once per call: nontemporal loads stream them
// past the caches (measured ~7.0 TB/s streaming-read ceiling on MI355X with
// the nontemporal hint, ~6.2 TB/s without).
__device__ __forceinline__ u32x4 ld16_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}

// Narrower streaming loads for pages of fewer than 16 slots.
__device__ __forceinline__ u32x2 ld8_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ uint32_t ld4_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(p));
}
__device__ __forceinline__ uint32_t ld2_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(p));
}
__device__ __forceinline__ uint32_t ld1_stream(const char* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const uint8_t*>(p));
}

// 16x16x32: A and B hold 8 consecutive k values per lane.
template <int QT>
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (QT == kF16) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// 16x16x16: A and B hold 4 consecutive k values per lane (PV over the 16 keys
// of one sub-tile in the half-step path).
template <int QT>
__device__ __forceinline__ f32x4 mfma16(u32x2 a, u32x2 b, f32x4 c) {
  if constexpr (QT == kF16) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                 __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a),
                                                     __builtin_bit_cast(i16x4, b), c, 0, 0, 0);
  }
}

// The four softmax weights of a lane for one sub-tile (half-step path), as
// pack_p below.
template <int QT>
__device__ __forceinline__ void pack_p4(const float (&p)[4], u32x2& hi, u32x2& lo) {
  if constexpr (QT == kF16) {
    f16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (_Float16)p[e];
    hi = __builtin_bit_cast(u32x2, h);
    lo = u32x2{0, 0};
  } else {
    bf16x4 h, l;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (__bf16)p[e];
      l[e] = (__bf16)(p[e] - (float)h[e]);
    }
    hi = __builtin_bit_cast(u32x2, h);
    lo = __builtin_bit_cast(u32x2, l);
  }
}

// The eight softmax weights of a lane — keys 4*q4 + 0..3 of sub-tile 0, then
// of sub-tile 1 — as the B operand of a 16x16x32 product.  f16: one
// round-to-nearest per weight (at most 2^-11 relative).  bf16 keeps only 8
// bits, which costs up to 2^-9 of max|v| when a few keys dominate, so the
// weights are split as hi = rne(p), lo = rne(p - hi) and PV runs on both.
template <int QT>
__device__ __forceinline__ void pack_p(const float (&p)[8], u32x4& hi, u32x4& lo) {
  if constexpr (QT == kF16) {
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = (_Float16)p[e];
    hi = __builtin_bit_cast(u32x4, h);
    lo = u32x4{0, 0, 0, 0};
  } else {
    bf16x8 h, l;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      h[e] = (__bf16)p[e];
      l[e] = (__bf16)(p[e] - (float)h[e]);
    }
    hi = __builtin_bit_cast(u32x4, h);
    lo = __builtin_bit_cast(u32x4, l);
  }
}

// Four u8 codes (one dword) as four exact 16-bit values of the MFMA type,
// offset by kU8Bias<QT>.  f16: byte b placed under exponent 0x64 is the half
// 1024 + b, one byte permute per two codes; the 1024 is folded into the zero
// point by the caller.  bf16 has too few mantissa bits for that and goes
// through f32 without an offset.
template <int QT>
constexpr float kU8Bias = QT == kF16 ? 1024.f : 0.f;

template <int QT>
__device__ __forceinline__ u32x2 u8x4_to_16(uint32_t w) {
  if constexpr (QT == kF16) {
    return u32x2{__builtin_amdgcn_perm(0x64646464u, w, 0x04010400u),
                 __builtin_amdgcn_perm(0x64646464u, w, 0x04030402u)};
  } else {
    bf16x4 h;
#pragma unroll
    for (int e = 0; e < 4; ++e) h[e] = (__bf16)(float)((w >> (8 * e)) & 0xffu);
    return __builtin_bit_cast(u32x2, h);
  }
}

// Wait for this wavefront's LDS operations; the memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void wait_lgkmcnt0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// ---------------------------------------------------------------------------
// Cross-lane exchanges without LDS.  Each pairs every lane with one partner
// (an involution), so a reduction built from them leaves the same bits in
// every lane (a + b and b + a round alike).  DPP quad permutes and row
// mirrors stay inside a 16-lane row; gfx950's permlane swaps cross rows.
// v_permlane16_swap a, b exchanges a's odd rows with b's even rows, so with
// a = b = x it leaves a = rows (0,0,2,2) and b = rows (1,1,3,3) of x;
// v_permlane32_swap likewise leaves a = halves (0,0), b = (1,1).  Combining
// a and b then pairs each lane with lane ^ 16 or lane ^ 32.  The swaps are
// issued as inline asm on two tied registers: the compiler's builtins for
// them fold the swap of two equal operands into a copy, which is wrong
// across lanes.  The asm carries its own wait states (a VALU write of an
// operand needs two before a permlane swap reads it).
// ---------------------------------------------------------------------------
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15 - i within 16

__device__ __forceinline__ void swap16(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap32(uint32_t& a, uint32_t& b) {
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
template <typename F>
__device__ __forceinline__ float pair16(float v, F op) {
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  swap16(a, b);
  return op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
template <typename F>
__device__ __forceinline__ float pair32(float v, F op) {
  uint32_t a = __builtin_bit_cast(uint32_t, v), b = a;
  swap32(a, b);
  return op(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}
__device__ __forceinline__ float fmax_op(float a, float b) { return fmaxf(a, b); }
__device__ __forceinline__ float fmin_op(float a, float b) { return fminf(a, b); }
__device__ __forceinline__ float fadd_op(float a, float b) { return a + b; }

// v combined with lane ^ 16, then lane ^ 32 (the four lane groups of a row)
__device__ __forceinline__ float group_max(float v) {
  return pair32(pair16(v, fmax_op), fmax_op);
}
__device__ __forceinline__ float group_sum(float v) {
  return pair32(pair16(v, fadd_op), fadd_op);
}

// all 64 lanes
template <typename F>
__device__ __forceinline__ float wave_reduce(float v, F op) {
  v = op(v, __builtin_bit_cast(float, dpp_u32<kDppXor1>(__builtin_bit_cast(uint32_t, v))));
  v = op(v, __builtin_bit_cast(float, dpp_u32<kDppXor2>(__builtin_bit_cast(uint32_t, v))));
  v = op(v, __builtin_bit_cast(float, dpp_u32<kDppHalfMirror>(__builtin_bit_cast(uint32_t, v))));
  v = op(v, __builtin_bit_cast(float, dpp_u32<kDppMirror>(__builtin_bit_cast(uint32_t, v))));
  return pair32(pair16(v, op), op);
}
__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, fmax_op); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, fadd_op); }

// integer sum over all 64 lanes (exact, every lane gets it)
__device__ __forceinline__ int wave_sum_i32(int v) {
  v += (int)dpp_u32<kDppXor1>((uint32_t)v);
  v += (int)dpp_u32<kDppXor2>((uint32_t)v);
  v += (int)dpp_u32<kDppHalfMirror>((uint32_t)v);
  v += (int)dpp_u32<kDppMirror>((uint32_t)v);
  uint32_t a = (uint32_t)v, b = a;
  swap16(a, b);
  a = b = a + b;
  swap32(a, b);
  return (int)(a + b);
}
__device__ __forceinline__ int wave_max_i32(int v) {
  v = max(v, (int)dpp_u32<kDppXor1>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppXor2>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppHalfMirror>((uint32_t)v));
  v = max(v, (int)dpp_u32<kDppMirror>((uint32_t)v));
  uint32_t a = (uint32_t)v, b = a;
  swap16(a, b);
  a = b = (uint32_t)max((int)a, (int)b);
  swap32(a, b);
  return max((int)a, (int)b);
}

__device__ __forceinline__ float lo_f16(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[0];
}
__device__ __forceinline__ float hi_f16(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[1];
}

// Per-sequence decode shared by both kernels: the contract check and the
// step/segment ranges.  Keys of the sequence that any row reads lie in
// [lo0, ctx); steps are kKeysPerStep-key windows starting at base.
struct SeqInfo {
  int b0, T, L, ctx, lo0, base, n_steps;
  bool ok;
};

// rows: stacked query rows the kernel instance holds (G * T must fit).
// b0, b1: subsequence_begins[s], [s + 1]; L: past_lens[s].
__device__ __forceinline__ SeqInfo seq_decode(const SegmentArgs& a, int b0, int b1, int L, int rows) {
  SeqInfo q;
  q.b0 = b0;
  q.T = b1 - b0;
  q.L = L;
  q.ok = b0 >= 0 && b1 <= a.num_tokens && q.T >= 1 && q.T <= a.max_q && L >= 0 &&
         (int64_t)L + q.T <= a.max_ctx && a.G * q.T <= rows;
  q.ctx = L + q.T;
  q.lo0 = a.window > 0 ? max(0, L + 1 - a.window) : 0;
  q.base = (q.lo0 / kKeysPerStep) * kKeysPerStep;
  q.n_steps = q.ok ? (q.ctx - q.base + kKeysPerStep - 1) / kKeysPerStep : 0;
  return q;
}
__device__ __forceinline__ SeqInfo seq_info(const SegmentArgs& a, int s, int rows) {
  return seq_decode(a, a.sb[s], a.sb[s + 1], a.past_lens[s], rows);
}

// ceil(n / c) for 0 <= n < 2^26 and 1 <= c < 2^16, exact; rc = rcp(c).  A
// float estimate q0 of floor(m / c), m = n + c - 1, is within 60 of it; the
// remainder m - q0 c (exact in float) then gives the rest to within one,
// and one integer comparison settles it.
__device__ __forceinline__ int ceil_div_small(int n, int c, float rc) {
  const int m = n + c - 1;
  int q = (int)((float)m * rc);
  q += (int)floorf((float)(m - q * c) * rc);
  const int r = m - q * c;
  return q + (r >= c) - (r < 0);
}

// inclusive prefix sum over the 64 lanes: DPP row shifts inside each 16-lane
// row, then the totals of the rows before it (read from lanes 15, 31, 47)
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xf, 0xf, true);   // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xf, 0xf, true);   // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xf, 0xf, true);   // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xf, 0xf, true);   // row_shr:8
  const int r0 = __builtin_amdgcn_readlane(v, 15);
  const int r1 = __builtin_amdgcn_readlane(v, 31);
  const int r2 = __builtin_amdgcn_readlane(v, 47);
  const int row = (int)(threadIdx.x & (kWave - 1)) >> 4;
  return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

// ---------------------------------------------------------------------------
// Work list of a batch of 2 .. kWlSeqs sequences (the planner gives larger
// batches, and any batch whose sequences outnumber the target, fixed
// per-sequence segments: every sequence then has a chunk of its own
// whatever the chunk size, which is what those segments are).  Every
// sequence's steps are cut into chunks of C steps; C is the smallest size
// (not below the host's steps per segment, nor above what the LDS block-id
// table holds) whose chunks of all sequences fit the target count of
// workgroups per KV head, so one round of equal workgroups covers the batch
// however its lengths are spread.  A sequence that breaks the contract gets
// one chunk (it writes NaN partials).  Wavefront 0 of every workgroup loads
// the batch's metadata once into registers (lane-strided, one request per
// array) and computes C and the workgroup's chunk from them.  Wave-wide.
// ---------------------------------------------------------------------------
struct WorkList {
  int code[kWlCached];                 // steps; -1 breaks the contract; -2 past the batch
  int b0[kWlCached], b1[kWlCached], L[kWlCached];
  int P;                               // 64-lane groups holding sequences (uniform)
};
__device__ __forceinline__ WorkList wl_load(const SegmentArgs& a, int rows) {
  const int lane = threadIdx.x & (kWave - 1);
  WorkList w;
  w.P = min((a.num_seqs + kWave - 1) / kWave, kWlCached);
#pragma unroll
  for (int p = 0; p < kWlCached; ++p) {
    const int s = p * kWave + lane;
    const bool in = p < w.P && s < a.num_seqs;
    w.b0[p] = in ? a.sb[s] : 0;
    w.b1[p] = in ? a.sb[s + 1] : 0;
    w.L[p] = in ? a.past_lens[s] : 0;
  }
#pragma unroll
  for (int p = 0; p < kWlCached; ++p) {
    const SeqInfo q = seq_decode(a, w.b0[p], w.b1[p], w.L[p], rows);
    w.code[p] = p * kWave + lane >= a.num_seqs ? -2 : q.ok ? q.n_steps : -1;
  }
  return w;
}
__device__ __forceinline__ int wl_items(int code, int C, float rc) {
  return code >= 0 ? ceil_div_small(code, C, rc) : code == -1 ? 1 : 0;
}

// chunks of all sequences for chunk size C
__device__ __forceinline__ int wl_count(int C, const WorkList& w) {
  const float rc = __builtin_amdgcn_rcpf((float)C);
  int n = 0;
#pragma unroll
  for (int p = 0; p < kWlCached; ++p)
    if (p < w.P) n += wl_items(w.code[p], C, rc);
  return wave_sum_i32(n);
}

// sum over aligned groups of g lanes (g a power of two, uniform), every lane
// of a group left with its group's total
__device__ __forceinline__ int lane_group_sum(int v, int g) {
  if (g > 1) v += (int)dpp_u32<kDppXor1>((uint32_t)v);
  if (g > 2) v += (int)dpp_u32<kDppXor2>((uint32_t)v);
  if (g > 4) v += (int)dpp_u32<kDppHalfMirror>((uint32_t)v);
  if (g > 8) v += (int)dpp_u32<kDppMirror>((uint32_t)v);
  if (g > 16) {
    uint32_t x = (uint32_t)v, y = x;
    swap16(x, y);
    v = (int)(x + y);
  }
  if (g > 32) {
    uint32_t x = (uint32_t)v, y = x;
    swap32(x, y);
    v = (int)(x + y);
  }
  return v;
}

// The smallest C in [lo, hi] whose chunks number at most `target`, given
// that C = hi's do, for a batch of 2 .. 64 sequences (sequence i's code in
// lane i): the wavefront splits into groups of g lanes (the sequence count
// rounded up to a power of two), each holding a copy of the codes and
// testing one candidate, so each round cuts the range into 64 / g + 1
// parts instead of two.
__device__ __forceinline__ int wl_search_small(int lo, int hi, int target, int num_seqs, int code0) {
  const int lane = threadIdx.x & (kWave - 1);
  const int lg = 32 - __clz(num_seqs - 1);                  // log2 g
  const int g = 1 << lg;
  const int k = lane >> lg;                                 // this lane's candidate
  const int kn = kWave >> lg;                               // candidates per round
  const int code = __shfl(code0, lane & (g - 1), kWave);
  const float inv = 1.0f / (float)(kn + 1);
  while (lo < hi) {
    // kn non-decreasing candidates in [lo, hi - 1], about evenly spaced
    const int span = hi - lo;
    auto cand = [&](int kk) { return lo + min(span - 1, (int)((float)((kk + 1) * span) * inv)); };
    const int c = cand(k);
    const int n = lane_group_sum(wl_items(code, c, __builtin_amdgcn_rcpf((float)c)), g);
    const unsigned long long fits = __ballot(n <= target && (lane & (g - 1)) == 0);
    if (fits) {
      // the first fitting candidate; the one before it (a smaller C) did not fit
      const int kf = __builtin_ctzll(fits) >> lg;
      const int c_hi = cand(kf);
      if (kf > 0) lo = cand(kf - 1) + 1;
      hi = c_hi;
    } else {
      lo = cand(kn - 1) + 1;
    }
  }
  return lo;
}

__device__ __forceinline__ int wl_chunk(const SegmentArgs& a, const WorkList& w) {
  long long total = 0;
  int longest = 1;
#pragma unroll
  for (int p = 0; p < kWlCached; ++p) {
    const int st = max(w.code[p], 0);
    total += st;
    longest = max(longest, st);
  }
  // a lane's share of the total stays below 2^28 (kWlCached sequences of at
  // most 2^26 steps each): summed as 16-bit high and low parts, each of
  // whose totals fits 32 bits
  {
    const int hi = wave_sum_i32((int)(total >> 16));
    const int lo = wave_sum_i32((int)(total & 0xffff));
    total = ((long long)hi << 16) + lo;
  }
  longest = wave_max_i32(longest);
  // ceil(total / target): total < 2^53 and the quotient lies at least
  // 1 / target from an integer unless it is one, far more than its
  // rounding error, so the ceiling of the double quotient is exact
  const long long want = (long long)ceil((double)total / (double)a.target_items);
  int hi = max(1, min(longest, a.max_sps));               // a chunk's block ids fit LDS
  int lo = (int)min<long long>(max<long long>(a.steps_per_seg, want), hi);
  lo = max(lo, 1);
  if (wl_count(hi, w) > a.target_items) return hi;       // the fewest chunks possible
  if (w.P == 1) return wl_search_small(lo, hi, a.target_items, a.num_seqs, w.code[0]);
  while (lo < hi) {                                       // smallest C that fits
    const int mid = lo + (hi - lo) / 2;
    if (wl_count(mid, w) <= a.target_items) hi = mid; else lo = mid + 1;
  }
  return lo;
}

// The sequence holding chunk number `item` (in sequence order): its index,
// the chunk's index inside it, the sequence's chunk count and metadata;
// -1 when item is past the last chunk.
struct WlHit {
  int seq, chunk, items, b0, b1, L;
};
__device__ __forceinline__ WlHit wl_find(int C, int item, const WorkList& w) {
  const float rc = __builtin_amdgcn_rcpf((float)C);
  WlHit h{-1, 0, 0, 0, 0, 0};
  int base = 0;
#pragma unroll
  for (int p = 0; p < kWlCached; ++p) {
    if (p >= w.P) break;                                  // uniform
    const int items = wl_items(w.code[p], C, rc);
    const int inc = wave_incl_scan(items);
    const int excl = inc - items;
    const unsigned long long hit = __ballot(item >= base + excl && item < base + inc);
    if (hit) {
      const int l = __builtin_ctzll(hit);
      h.seq = p * kWave + l;
      h.chunk = item - base - __builtin_amdgcn_readlane(excl, l);
      h.items = __builtin_amdgcn_readlane(items, l);
      h.b0 = __builtin_amdgcn_readlane(w.b0[p], l);
      h.b1 = __builtin_amdgcn_readlane(w.b1[p], l);
      h.L = __builtin_amdgcn_readlane(w.L[p], l);
      return h;
    }
    base += __builtin_amdgcn_readlane(inc, kWave - 1);
  }
  return h;
}

// ---------------------------------------------------------------------------
// Segment kernel.  QT: dtype of q (and of the MFMA operands); KV: cache dtype
// (QT, or kU8 for codes with per-token f16 scale and zero point); RB: 16-row
// blocks of stacked query rows (G * T <= 16 * RB): each K/V operand a step
// loads (and, for u8, converts) feeds one MFMA per row block; HR: register
// sets of the half-step path (0: whole steps); PL: page layout (kPagesTiled,
// or kPagesRowMajor: every page [slot][d] for K and V).
// ---------------------------------------------------------------------------
template <int QT, int KV, int D, int BS, int NW, int WPE, int RB, int HR, int PL>
__global__ __launch_bounds__(NW * kWave) __attribute__((amdgpu_waves_per_eu(WPE)))
void pa_segment(SegmentArgs a) {
  constexpr bool U8 = KV == kU8;
  constexpr int EB = U8 ? 1 : 2;                  // bytes per cached element
  constexpr int QC = D / 32;                      // 16x16x32 k-chunks of the QK contraction
  constexpr int LK = U8 ? D / 64 : D / 32;        // 1 KB K loads per 16-slot sub-tile
  constexpr int LV = LK;                          // 1 KB V loads per sub-tile
  constexpr int DT = D / 16;                      // 16-wide d tiles of O^T
  constexpr int OSTRIDE = D + 4;                  // padded LDS row of the merge buffer
  constexpr int ROWS = kRows * RB;                // stacked rows this instance holds
  static_assert((BS % 16 == 0 || BS == 1 || BS == 2 || BS == 4 || BS == 8) && kKeysPerStep == 32,
                "two 16-slot sub-tiles per step, within one page or across 16 / BS pages");
  constexpr int kSegSlots = seg_block_slots(BS);
  __shared__ int s_bt[kSegSlots];
  __shared__ float s_m[NW][ROWS];
  __shared__ float s_l[NW][ROWS];
  __shared__ int s_bad;
  // Pages of fewer than 16 slots: K (and for 1 or 2 slots, V) is loaded as
  // whole page rows (1 KB per instruction) and turned into the MFMA operand
  // layout through a per-wavefront LDS area, K first, then V: each
  // sub-tile's 16/BS pages, page-major, each padded by 16 B against bank
  // conflicts.  Row-major pages hold V [slot][d], while the PV operand wants
  // four keys of one d per lane: their V sub-tiles (16 rows, each padded by
  // 16 B) take the same path at every page size.  Row-major K of a 16-slot
  // sub-tile is loaded straight into the operand order (16 B of the lane's
  // slot row).
  constexpr bool ROWV = PL == kPagesRowMajor;
  constexpr bool WIDE_K = BS < 16;
  constexpr bool WIDE_V = BS <= 2 || ROWV;
  constexpr bool STAGE = WIDE_K || WIDE_V;
  constexpr int kPageBytes = BS * D * EB;                 // one page of one KV head (K or V)
  constexpr int kPagePad = kPageBytes + 16;
  constexpr int kRowPad = D * EB + 16;                    // staged row of a 16-slot sub-tile
  constexpr int kVtTau = BS < 16 ? (16 / BS) * kPagePad : 16 * kRowPad;   // one sub-tile
  // With row-major pages the staging area and the merge buffer share LDS
  // (used one after the other, a barrier between).
  constexpr bool ALIAS = ROWV;
  constexpr size_t kSoBytes = (size_t)NW * ROWS * OSTRIDE * 4;
  constexpr size_t kVtBytes = STAGE ? (size_t)NW * 2 * kVtTau : 16;
  __shared__ __attribute__((aligned(16))) char s_obuf[ALIAS && kVtBytes > kSoBytes ? kVtBytes : kSoBytes];
  __shared__ __attribute__((aligned(16))) char s_vtbuf[ALIAS ? 16 : kVtBytes];
  auto& s_o = *reinterpret_cast<float (*)[NW][ROWS][OSTRIDE]>(s_obuf);
  char* const s_vt = ALIAS ? s_obuf : s_vtbuf;
  // byte of (sub-tile slot s, dim d) in a staged sub-tile: K pages are
  // row-major within the page in both layouts, V pages too with row-major
  // pages, d-major for tiled pages of fewer than 16 slots
  auto staged_k = [&](int s, int d) {
    if constexpr (BS >= 16) return s * kRowPad + d * EB;
    else return (s / BS) * kPagePad + ((s % BS) * D + d) * EB;
  };
  auto staged_v = [&](int s, int d) {
    if constexpr (BS >= 16 || ROWV) return staged_k(s, d);
    else return (s / BS) * kPagePad + (d * BS + s % BS) * EB;
  };
  // staging offset of byte L of a sub-tile loaded as rows (1 KB per load)
  auto stage_off = [&](int L) {
    if constexpr (BS >= 16) return (L / (D * EB)) * kRowPad + L % (D * EB);
    else return (L / kPageBytes) * kPagePad + L % kPageBytes;
  };

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int n16 = lane & 15;          // stacked query row owned by this lane (in each row block)
  const int q4 = lane >> 4;           // lane group

  // Workgroup 0 checks subsequence_begins as a whole (starts at 0, never
  // decreases, ends at num_tokens): each wavefront writes its verdict on its
  // share of the entries, every call, so the combine kernel reads NW words
  // instead of scanning the batch.  The loads go out with the workgroup's
  // own metadata loads.
  static_assert(NW < 64, "one header word per wavefront");
  if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0) {
    bool bad = false;
#pragma unroll 4
    for (int i = threadIdx.x; i < a.num_seqs; i += NW * kWave) bad |= a.sb[i] > a.sb[i + 1];
    if (threadIdx.x == 0) bad |= a.sb[0] != 0 || a.sb[a.num_seqs] != a.num_tokens;
    const bool wave_bad = __any(bad);
    if (lane == 0) a.sb_check[wave] = wave_bad ? 1 : 0;
  }
  // Fixed segments (one sequence, or a batch of more sequences than the
  // work list takes): grid (Hkv, num_seqs, S) with segment j = S - 1 -
  // blockIdx.z.  Work-list mode (a small batch): grid (Hkv, 1, chunks), the
  // sequence and steps of chunk blockIdx.z taken from the work list.
  const int h = blockIdx.x;
  int s, j, st_begin, st_cap, wl_items = 0;
  WlHit wl_hit{};
  if (!a.worklist) {
    s = blockIdx.y;
    j = a.S - 1 - (int)blockIdx.z;
    // Segment j owns steps [j*N/S, (j+1)*N/S) of the N steps planned on the
    // host: segment lengths differ by at most one step.
    st_begin = (int)(((int64_t)j * a.n_steps) / a.S);
    st_cap = (int)(((int64_t)(j + 1) * a.n_steps) / a.S);
  } else {
    // wavefront 0 alone searches (its SIMD partner waits at the barrier
    // instead of competing for issue slots with the same work) and hands
    // the chunk to the others through LDS
    __shared__ int s_wl[7];
    if (wave == 0) {
      const WorkList wl = wl_load(a, ROWS);
      const int C = wl_chunk(a, wl);
      const WlHit hit = wl_find(C, (int)blockIdx.z, wl);
      if (lane == 0) {
        s_wl[0] = hit.seq;
        s_wl[1] = hit.chunk;
        s_wl[2] = hit.items;
        s_wl[3] = hit.b0;
        s_wl[4] = hit.b1;
        s_wl[5] = hit.L;
        s_wl[6] = C;
      }
    }
    __syncthreads();
    wl_hit = WlHit{s_wl[0], s_wl[1], s_wl[2], s_wl[3], s_wl[4], s_wl[5]};
    const int C = s_wl[6];
    s = wl_hit.seq;
    if (s < 0) return;                                        // past the last chunk (uniform)
    j = wl_hit.chunk;
    wl_items = wl_hit.items;
    st_begin = j * C;
    st_cap = st_begin + C;
  }
  const int32_t* bt_row = a.bt + (size_t)s * a.mbps;

  // Full-causal layers with a fixed segment grid: segment j's block range
  // does not depend on the sequence's length, so its block ids are
  // requested together with the sequence metadata — one memory round trip
  // before the first KV load instead of two.  The loads stay inside the
  // block-table row; ids of blocks past the sequence are never used.
  constexpr int kSlots = (kSegSlots + NW * kWave - 1) / (NW * kWave);
  int spec_id[kSlots];
  const int spec_lo = (st_begin * kKeysPerStep) / BS;
  const bool spec = a.window == 0 && !a.worklist;
  const int spec_n = spec ? min(a.mbps - spec_lo, (a.steps_per_seg * kKeysPerStep) / BS + 1) : 0;
#pragma unroll
  for (int k = 0; k < kSlots; ++k) {
    const int x = threadIdx.x + k * NW * kWave;
    spec_id[k] = x < spec_n ? bt_row[spec_lo + x] : 0;
  }

  const SeqInfo si = a.worklist ? seq_decode(a, wl_hit.b0, wl_hit.b1, wl_hit.L, ROWS)
                                : seq_info(a, s, ROWS);
  // Direct calls (one segment): output rows [t0, t1) x this KV head's q
  // heads become NaN (a sequence that breaks the contract, a row with no key)
  auto nan_rows = [&](int t0, int t1) {
    constexpr int V8 = D / 8;                                 // 16-byte pieces per row
    const uint16_t nan1 = QT == kF16 ? 0x7E00u : 0x7FC0u;
    const uint32_t nan2 = 0x10001u * nan1;
    const u32x4 nan8 = {nan2, nan2, nan2, nan2};
    for (int x = threadIdx.x; x < (t1 - t0) * a.G * V8; x += NW * kWave) {
      const int y = x / V8;
      const size_t row = (size_t)(t0 + y / a.G) * a.Hq + h * a.G + y % a.G;
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + row * D + (x % V8) * 8;
      *reinterpret_cast<u32x4*>(dst) = nan8;
    }
  };
  if (!si.ok) {
    // A sequence that breaks the contract: its partials for this segment
    // become NaN (for the tokens it claims that exist), so the combine turns
    // its rows into NaN without re-checking the sequence; a direct call
    // writes NaN rows.
    if (j == 0 && h == 0 && threadIdx.x == 0) atomicExch(a.status, kDeviceContract);
    const int t0 = min(max(si.b0, 0), a.num_tokens);
    const int t1 = min(max(si.b0 + si.T, t0), a.num_tokens);
    if (a.direct) {
      nan_rows(t0, t1);
      return;
    }
    // work-list mode: the sequence's only chunk marks all its slots
    const int nj = a.worklist ? a.S : 1;
    for (int x = threadIdx.x; x < (t1 - t0) * a.G * nj; x += NW * kWave) {
      const int jj = a.worklist ? x % nj : j, y = x / nj;
      const size_t row = ((size_t)(t0 + y / a.G) * a.Hq + h * a.G + y % a.G) * a.S + jj;
      a.ws_ml[row * 2 + 0] = NAN;
      a.ws_ml[row * 2 + 1] = 0.f;
    }
    return;
  }
  if (a.worklist && j == 0) {
    // slots past the sequence's chunks hold no partial: mark them empty so
    // the combine reads all S slots without knowing the chunk size
    const int R0 = a.G * si.T, nj = a.S - wl_items;
    for (int x = threadIdx.x; x < R0 * nj; x += NW * kWave) {
      const int r = x / nj, jj = wl_items + x % nj;
      const size_t row = ((size_t)(si.b0 + r % si.T) * a.Hq + h * a.G + r / si.T) * a.S + jj;
      a.ws_ml[row * 2 + 0] = -INFINITY;
      a.ws_ml[row * 2 + 1] = 0.f;
    }
  }
  const int T = si.T;
  const int R = a.G * T;
  const int st_end = min(si.n_steps, st_cap);
  if (st_begin >= st_end) {
    // no key of this sequence falls in segment j: an empty partial, so the
    // combine can read all S partials without knowing the sequence (a
    // direct call's only segment: rows with no key, NaN as the combine
    // would make them)
    if (a.direct) {
      nan_rows(si.b0, si.b0 + T);
      return;
    }
    if (threadIdx.x < R) {
      const int r = threadIdx.x;
      const size_t row = ((size_t)(si.b0 + r % T) * a.Hq + h * a.G + r / T) * a.S + j;
      a.ws_ml[row * 2 + 0] = -INFINITY;
      a.ws_ml[row * 2 + 1] = 0.f;
    }
    return;
  }

  // Stage the segment's block ids in LDS.  Only pages holding a key in
  // [lo0, ctx) are checked and ever dereferenced.
  const int key_lo = si.base + st_begin * kKeysPerStep;
  const int blk_lo = key_lo / BS;
  const int blk_last = (min(si.ctx, si.base + st_end * kKeysPerStep) - 1) / BS;
  if (threadIdx.x == 0) s_bad = 0;
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kSlots; ++k) {
    const int x = threadIdx.x + k * NW * kWave;
    if (x <= blk_last - blk_lo) {
      const int b = blk_lo + x;
      int id = 0;
      if ((b + 1) * BS > si.lo0) {
        id = spec ? spec_id[k] : bt_row[b];
        if ((unsigned)id >= (unsigned)a.num_blocks) {
          s_bad = 1;
          id = 0;
        }
      }
      s_bt[x] = id;
    }
  }

  // Stacked rows: r = g*T + i for q head h*G + g and token b0 + i; lane row
  // n16 of row block rb is r = 16*rb + n16.  Rows past G*T are padding that
  // no one reads back (they compute on a real token's q, so stay finite).
  // Row r sees cache position t when t >= lo_r and, for t >= L (the new
  // tokens), bit t - L of its mask vis_r is set: causal rows see new tokens
  // 0..i; a tree row sees the tokens its word names, itself always.
  bool row_ok[RB];
  int qh[RB], tok[RB], lo_r[RB];
  uint32_t vis_r[RB];
  const uint32_t tmask = T >= 32 ? 0xffffffffu : (1u << T) - 1u;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int r = rb * kRows + n16;
    row_ok[rb] = r < R;
    const int g = row_ok[rb] ? r / T : 0;
    const int i = row_ok[rb] ? r % T : T - 1;
    qh[rb] = h * a.G + g;
    tok[rb] = si.b0 + i;                                      // padded rows: a real token
    lo_r[rb] = a.window > 0 ? max(0, si.L + i + 1 - a.window) : 0;
    vis_r[rb] = (2u << i) - 1u;                               // causal: tokens 0..i
  }
  if (a.tree) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      const int i = tok[rb] - si.b0;
      vis_r[rb] = (a.tree[tok[rb]] & tmask) | (1u << i);
    }
  }
  const int lo_max = a.window > 0 ? max(0, si.ctx - a.window) : 0;
  // a step is interior when every row sees all of its keys: past keys only
  // for tree rows; for causal rows key L too (row 0 sees it)
  const int all_see = si.L + (a.tree ? 0 : 1);

  // B operand of the QK product: lane (row, group q4) holds, for k-chunk c,
  // the 8 d values the K sub-tile load puts in the same lane group:
  // d = c*32 + q4*8 + 0..7 (u8: chunk 2*c2 + half: d = c2*64 + q4*16 + half*8 + 0..7).
  u32x4 qreg[RB][QC];
  float qsum[RB];                                             // u8: sum of this lane's q values
  // Issued after the wavefront's first K loads (not before the barrier that
  // publishes the block ids), so the first KV request does not wait a memory
  // round trip for q.
  auto load_q = [&]() {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      qsum[rb] = 0.f;
      const char* qp = reinterpret_cast<const char*>(a.q) + ((size_t)tok[rb] * a.Hq + qh[rb]) * D * 2;
#pragma unroll
      for (int c = 0; c < QC; ++c) {
        const int d0 = U8 ? (c / 2) * 64 + q4 * 16 + (c % 2) * 8 : c * 32 + q4 * 8;
        const u32x4 v = ld16(qp + d0 * 2);
        qreg[rb][c] = row_ok[rb] ? v : u32x4{0, 0, 0, 0};
      }
    }
  };
  // u8: the row sum of q, taken once the first KV loads are in flight.
  auto finish_q = [&]() {
    if constexpr (U8) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
        for (int c = 0; c < QC; ++c) {
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            if constexpr (QT == kF16) {
              qsum[rb] += lo_f16(qreg[rb][c][w]) + hi_f16(qreg[rb][c][w]);
            } else {
              qsum[rb] += __builtin_bit_cast(float, qreg[rb][c][w] << 16) +
                          __builtin_bit_cast(float, qreg[rb][c][w] & 0xffff0000u);
            }
          }
        }
        qsum[rb] = group_sum(qsum[rb]);
      }
    }
  };
  __syncthreads();

  const char* kb = reinterpret_cast<const char*>(a.k);
  const char* vb = reinterpret_cast<const char*>(a.v);
  const char* kszb = reinterpret_cast<const char*>(a.ksz);
  const char* vszb = reinterpret_cast<const char*>(a.vsz);
  const int Hkv = a.Hkv;

  // Registers of one step (two 16-slot sub-tiles tau): K and V loads, and
  // for u8 the (scale, zero point) pairs of this lane group's 4 keys.
  struct Step {
    u32x4 k[2][LK];
    u32x4 v[2][LV];
    u32x4 ks[2], vs[2];
  };

  // Every load is issued unconditionally: a sub-tile holding no key of
  // [lo0, ctx) reads the segment's first page instead (always a valid
  // address) and is masked out in compute_step.  Branch-free loads keep the
  // outstanding-load count static, so the compiler's waits inside a step's
  // math are for exactly the registers they need.
  // Pages of 1, 2, 4 or 8 slots: K pages are row-major [slot][d] and V pages
  // d-major [d][slot], so each lane gathers its own operand pieces: the K row
  // of its slot (the same 16 B chunks a tiled sub-tile load delivers), and
  // for V the 4 consecutive slots of its lane group at each of its d, which
  // lie in one page when BS >= 4 (one 8 B load), else in 16 / BS ... pages.
  // Keys outside [lo0, ctx) read the segment's first page, as below.
  auto load_step_small = [&](int st, Step& r) {
    const int key0 = si.base + st * kKeysPerStep;
    // keys [t, t + n) of one page: its id and t's slot, or the segment's
    // first page when none of them lies in [lo0, ctx) (a piece that is only
    // partly inside reads its real page; its outside keys are masked later)
    auto page_row = [&](int t, int n, int& pg, int& row) {
      const bool present = t < si.ctx && t + n > si.lo0;
      pg = s_bt[present ? t / BS - blk_lo : 0];
      row = present ? t % BS : 0;
    };
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const int t0 = key0 + tau * 16;
      {
        // K as whole page rows: load c covers bytes [1024 c, 1024 c + 1024)
        // of the sub-tile's pages laid end to end
        static_assert(16 * D * EB == LK * 1024, "one 1 KB load per register of the step");
#pragma unroll
        for (int c = 0; c < LK; ++c) {
          const int L = c * 1024 + lane * 16;
          int wpg, wrow;                                      // wrow is 0: pages start at 16-slot bounds
          page_row(t0 + (L / kPageBytes) * BS, BS, wpg, wrow);
          r.k[tau][c] = ld16_stream(kb + ((size_t)wpg * Hkv + h) * kPageBytes + L % kPageBytes);
        }
      }
      constexpr int NP = BS >= 4 ? 1 : 4 / BS;                // pages holding the 4 slots
      constexpr int SP = 4 / NP;                              // slots per piece
      int pg[NP], row[NP];
#pragma unroll
      for (int pc = 0; pc < NP; ++pc) page_row(t0 + q4 * 4 + pc * SP, SP, pg[pc], row[pc]);
      // element (slot row[pc] .. + SP, d) of piece pc
      auto vaddr = [&](int pc, int d) {
        return vb + ((((size_t)pg[pc] * Hkv + h) * BS * D) + (size_t)d * BS + row[pc]) * EB;
      };
      if constexpr (WIDE_V) {
        // load c covers bytes [1024 c, 1024 c + 1024) of the sub-tile's pages
        // laid end to end: lane i reads 16 B of page (1024 c + 16 i) / page size
        static_assert(16 * D * EB == LV * 1024, "one 1 KB load per register of the step");
#pragma unroll
        for (int c = 0; c < LV; ++c) {
          const int L = c * 1024 + lane * 16;
          int wpg, wrow;                                      // wrow is 0: pages start at 16-slot bounds
          page_row(t0 + (L / kPageBytes) * BS, BS, wpg, wrow);
          r.v[tau][c] = ld16_stream(vb + ((size_t)wpg * Hkv + h) * kPageBytes + L % kPageBytes);
        }
      }
      if constexpr (U8) {
#pragma unroll
        for (int c = 0; c < (WIDE_V ? 0 : LV); ++c) {
#pragma unroll
          for (int jd = 0; jd < 4; ++jd) {
            const int d = c * 64 + jd * 16 + n16;
            uint32_t w;
            if constexpr (NP == 1) w = ld4_stream(vaddr(0, d));
            else if constexpr (NP == 2) w = ld2_stream(vaddr(0, d)) | (ld2_stream(vaddr(1, d)) << 16);
            else
              w = ld1_stream(vaddr(0, d)) | (ld1_stream(vaddr(1, d)) << 8) |
                  (ld1_stream(vaddr(2, d)) << 16) | (ld1_stream(vaddr(3, d)) << 24);
            r.v[tau][c][jd] = w;
          }
        }
        size_t so[NP];                                        // (scale, zero point) offsets
#pragma unroll
        for (int pc = 0; pc < NP; ++pc) so[pc] = (((size_t)pg[pc] * Hkv + h) * BS + row[pc]) * 4;
        u32x4 ks, vs;
        if constexpr (NP == 1) {
          ks = ld16_stream(kszb + so[0]);
          vs = ld16_stream(vszb + so[0]);
        } else if constexpr (NP == 2) {
          const u32x2 k0 = ld8_stream(kszb + so[0]), k1 = ld8_stream(kszb + so[1]);
          const u32x2 v0 = ld8_stream(vszb + so[0]), v1 = ld8_stream(vszb + so[1]);
          ks = u32x4{k0[0], k0[1], k1[0], k1[1]};
          vs = u32x4{v0[0], v0[1], v1[0], v1[1]};
        } else {
#pragma unroll
          for (int pc = 0; pc < 4; ++pc) {
            ks[pc] = ld4_stream(kszb + so[pc]);
            vs[pc] = ld4_stream(vszb + so[pc]);
          }
        }
        r.ks[tau] = ks;
        r.vs[tau] = vs;
      } else {
#pragma unroll
        for (int dp = 0; dp < (WIDE_V ? 0 : LV); ++dp) {
          u32x2 half[2];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int d = dp * 32 + hh * 16 + n16;
            if constexpr (NP == 1) {
              half[hh] = ld8_stream(vaddr(0, d));
            } else if constexpr (NP == 2) {
              half[hh] = u32x2{ld4_stream(vaddr(0, d)), ld4_stream(vaddr(1, d))};
            } else {
              half[hh] = u32x2{ld2_stream(vaddr(0, d)) | (ld2_stream(vaddr(1, d)) << 16),
                               ld2_stream(vaddr(2, d)) | (ld2_stream(vaddr(3, d)) << 16)};
            }
          }
          r.v[tau][dp] = u32x4{half[0][0], half[0][1], half[1][0], half[1][1]};
        }
      }
    }
  };

  // 16-slot pages: the K loads of both sub-tiles, then (between: the q rows
  // on a wavefront's first step) the V and scale loads.
  auto tile_of = [&](int st, int tau) {
    const int t0 = si.base + st * kKeysPerStep + tau * 16;    // first key of the sub-tile
    const bool present = t0 < si.ctx && t0 + 16 > si.lo0;
    const int page = __builtin_amdgcn_readfirstlane(s_bt[present ? t0 / BS - blk_lo : 0]);
    const int sub = present ? (t0 % BS) / 16 : 0;
    return ((size_t)page * Hkv + h) * BS + (size_t)sub * 16;  // first slot row of the sub-tile
  };
  auto load_k = [&](int st, Step& r) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      if constexpr (ROWV) {
        // row-major: lane (slot n16, group q4) reads 16 B of its slot's row
        const char* kp = kb + (tile_of(st, tau) + n16) * D * EB;
#pragma unroll
        for (int c = 0; c < LK; ++c)
          r.k[tau][c] = ld16_stream(kp + (U8 ? c * 64 + q4 * 16 : c * 32 + q4 * 8) * EB);
      } else {
        const char* kp = kb + tile_of(st, tau) * D * EB + lane * 16;
#pragma unroll
        for (int c = 0; c < LK; ++c) r.k[tau][c] = ld16_stream(kp + c * 1024);
      }
    }
  };
  auto load_v = [&](int st, Step& r) {
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const size_t row0 = tile_of(st, tau);
      const char* vp = vb + row0 * D * EB + lane * 16;
#pragma unroll
      for (int c = 0; c < LV; ++c) r.v[tau][c] = ld16_stream(vp + c * 1024);
      if constexpr (U8) {
        const size_t srow = (row0 + q4 * 4) * 4;
        r.ks[tau] = ld16_stream(kszb + srow);
        r.vs[tau] = ld16_stream(vszb + srow);
      }
    }
  };
  auto load_step = [&](int st, Step& r, bool with_q) {
    if constexpr (BS < 16) {
      load_step_small(st, r);
      if (with_q) load_q();
    } else {
      load_k(st, r);
      if (with_q) load_q();
      load_v(st, r);
    }
  };

  f32x4 o[RB][DT];
  float m_run[RB];                    // running max (log2 units) of this lane's row
  float l_run[RB];                    // this lane's share of the running sum
  float c_run[RB];                    // u8: this lane's share of sum p * s_v * zp_v
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[rb][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
    c_run[rb] = 0.f;
  }

  // Pages of fewer than 16 slots: the step's K (and for 1 or 2 slots its V),
  // loaded as page rows, through LDS into the operand order of a tiled
  // sub-tile (K: 8 or 16 d of the lane's slot; V: for each d, the 4 keys
  // 4*q4 .. 4*q4+3 of the lane group).  The area is this wavefront's own;
  // the waits keep the reads after the writes and the compiler from moving
  // LDS accesses across them.
  auto to_operands = [&](Step& r) {
    char* vt = s_vt + wave * 2 * kVtTau;
    if constexpr (WIDE_K) {
      // K: lane (slot n16, group q4) takes the 16 B of its slot's row that a
      // tiled sub-tile load would give it
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
        for (int c = 0; c < LK; ++c)
          *reinterpret_cast<u32x4*>(vt + tau * kVtTau + stage_off(c * 1024 + lane * 16)) = r.k[tau][c];
      }
      wait_lgkmcnt0();
#pragma unroll
      for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
        for (int c = 0; c < LK; ++c) {
          const int d0 = U8 ? c * 64 + q4 * 16 : c * 32 + q4 * 8;
          r.k[tau][c] = *reinterpret_cast<const u32x4*>(vt + tau * kVtTau + staged_k(n16, d0));
        }
      }
    }
    if constexpr (!WIDE_V) return;
    wait_lgkmcnt0();                                          // K read back before V overwrites it
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
#pragma unroll
      for (int c = 0; c < LV; ++c)
        *reinterpret_cast<u32x4*>(vt + tau * kVtTau + stage_off(c * 1024 + lane * 16)) = r.v[tau][c];
    }
    wait_lgkmcnt0();
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      const char* base = vt + tau * kVtTau;
      auto at = [&](int s, int d) { return base + staged_v(s, d); };
      const int s0 = 4 * q4;
      if constexpr (U8) {
#pragma unroll
        for (int c = 0; c < LV; ++c) {
#pragma unroll
          for (int jd = 0; jd < 4; ++jd) {
            const int d = c * 64 + jd * 16 + n16;
            uint32_t w;
            if constexpr (BS == 2 && !ROWV)                   // two adjacent slots per read
              w = *reinterpret_cast<const uint16_t*>(at(s0, d)) |
                  ((uint32_t)*reinterpret_cast<const uint16_t*>(at(s0 + 2, d)) << 16);
            else
              w = (uint32_t)*reinterpret_cast<const uint8_t*>(at(s0, d)) |
                  ((uint32_t)*reinterpret_cast<const uint8_t*>(at(s0 + 1, d)) << 8) |
                  ((uint32_t)*reinterpret_cast<const uint8_t*>(at(s0 + 2, d)) << 16) |
                  ((uint32_t)*reinterpret_cast<const uint8_t*>(at(s0 + 3, d)) << 24);
            r.v[tau][c][jd] = w;
            // row-major pages: four byte reads per word; keep the scheduler
            // from hoisting all of a step's reads (their temporaries spill)
            if constexpr (ROWV) __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
#pragma unroll
        for (int dp = 0; dp < LV; ++dp) {
          uint32_t w[4];
#pragma unroll
          for (int hh = 0; hh < 2; ++hh) {
            const int d = dp * 32 + hh * 16 + n16;
            if constexpr (BS == 2 && !ROWV) {                 // two adjacent slots per read
              w[2 * hh] = *reinterpret_cast<const uint32_t*>(at(s0, d));
              w[2 * hh + 1] = *reinterpret_cast<const uint32_t*>(at(s0 + 2, d));
            } else {
              w[2 * hh] = (uint32_t)*reinterpret_cast<const uint16_t*>(at(s0, d)) |
                          ((uint32_t)*reinterpret_cast<const uint16_t*>(at(s0 + 1, d)) << 16);
              w[2 * hh + 1] = (uint32_t)*reinterpret_cast<const uint16_t*>(at(s0 + 2, d)) |
                              ((uint32_t)*reinterpret_cast<const uint16_t*>(at(s0 + 3, d)) << 16);
            }
          }
          r.v[tau][dp] = u32x4{w[0], w[1], w[2], w[3]};
          if constexpr (ROWV) __builtin_amdgcn_sched_barrier(0);
        }
      }
    }
  };

  auto compute_step = [&](int st, Step& r) {
    if constexpr (STAGE) to_operands(r);
    const int key0 = si.base + st * kKeysPerStep;
    // S^T for both sub-tiles: lane (row, q4) gets keys key0 + 16*tau + 4*q4 + 0..3
    float sv[RB][8];
#pragma unroll
    for (int tau = 0; tau < 2; ++tau) {
      // two interleaved accumulation chains per row block: no MFMA waits on
      // the one before
      f32x4 acc0[RB], acc1[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc0[rb] = acc1[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (U8) {
#pragma unroll
        for (int c2 = 0; c2 < LK; ++c2) {
          const u32x4 w = r.k[tau][c2];
          const u32x2 a0 = u8x4_to_16<QT>(w[0]), a1 = u8x4_to_16<QT>(w[1]);
          const u32x2 a2 = u8x4_to_16<QT>(w[2]), a3 = u8x4_to_16<QT>(w[3]);
          const u32x4 k0 = {a0[0], a0[1], a1[0], a1[1]}, k1 = {a2[0], a2[1], a3[0], a3[1]};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc0[rb] = mfma32<QT>(k0, qreg[rb][2 * c2], acc0[rb]);
            acc1[rb] = mfma32<QT>(k1, qreg[rb][2 * c2 + 1], acc1[rb]);
          }
        }
        // q.(u - zp) * s = s * (q.(u + bias) - (zp + bias) * sum(q))
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const f32x4 acc = acc0[rb] + acc1[rb];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sk = lo_f16(r.ks[tau][e]), zk = hi_f16(r.ks[tau][e]) + kU8Bias<QT>;
            sv[rb][tau * 4 + e] = sk * (acc[e] - zk * qsum[rb]) * a.scale_log2;
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < QC; c += 2) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc0[rb] = mfma32<QT>(r.k[tau][c], qreg[rb][c], acc0[rb]);
            if (c + 1 < QC) acc1[rb] = mfma32<QT>(r.k[tau][c + 1], qreg[rb][c + 1], acc1[rb]);
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const f32x4 acc = acc0[rb] + acc1[rb];
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[rb][tau * 4 + e] = acc[e] * a.scale_log2;
        }
      }
    }

    // Keys outside [lo0, ctx) may hold anything, NaN included: their logits
    // become -inf and, since 0 * NaN is not 0, their V (or u8 scale) never
    // reaches the PV product.
    const bool interior = key0 >= lo_max && key0 + kKeysPerStep <= all_see;
    bool kvalid[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) kvalid[e] = true;
    if (!interior) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int t = key0 + (e >> 2) * 16 + q4 * 4 + (e & 3);
        kvalid[e] = t >= si.lo0 && t < si.ctx;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const bool seen = t >= lo_r[rb] && (t < si.L || (t < si.ctx && ((vis_r[rb] >> (t - si.L)) & 1u)));
          sv[rb][e] = seen ? sv[rb][e] : -INFINITY;
        }
      }
    }

    u32x4 pb_hi[RB], pb_lo[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = sv[rb][0];
#pragma unroll
      for (int e = 1; e < 8; ++e) mx = fmaxf(mx, sv[rb][e]);
      mx = group_max(mx);
      // Lazy rescaling: weights are taken relative to a reference max m_run
      // that only moves when a logit passes it by more than 2^kRescaleLog2,
      // so weights stay <= 256 and the O rescale runs in few steps.  The
      // branch is wave-uniform.
      const bool need = mx > m_run[rb] + kRescaleLog2;
      if (__any(need)) {
        const float m_new = need ? mx : m_run[rb];
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - (m_new == -INFINITY ? 0.f : m_new));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rb][dt] *= alpha;
        l_run[rb] *= alpha;
        c_run[rb] *= alpha;
        m_run[rb] = m_new;
      }
      const float m_use = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
      float p[8];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sv[rb][e] - m_use);
        psum += p[e];
      }
      l_run[rb] += psum;

      if constexpr (U8) {
        // (u - zp) * s folded: the codes (offset by the bias) are multiplied
        // by P' = p * s_v, and sum(P' * (zp_v + bias)) is subtracted from
        // every d at the end.  With f16 weights the sum uses P' as rounded
        // for the MFMA, so the bias cancels exactly.
        float csum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t w = r.vs[e >> 2][e & 3];
          float sp = kvalid[e] ? p[e] * lo_f16(w) : 0.f;
          if constexpr (QT == kF16) sp = (float)(_Float16)sp;
          csum += kvalid[e] ? sp * (hi_f16(w) + kU8Bias<QT>) : 0.f;   // zp of a key outside may be NaN
          p[e] = sp;
        }
        c_run[rb] += csum;
      }
      pack_p<QT>(p, pb_hi[rb], pb_lo[rb]);
    }
    // PV, O^T[d, r] += V^T[d, key] P^T[key, r] with one 16x16x32 product per
    // 16-wide d tile and row block: the A operand of lane (d, q4) is V of
    // keys 4*q4 + 0..3 of both sub-tiles, the k order of the weights above.
    // The loaded V registers are never modified: in a boundary step the
    // f16/bf16 V of a key outside [lo0, ctx) is cleared as it is consumed
    // (u8 codes are finite; their P' is already 0).
    auto pv = [&](auto masked) {
      u32x2 vmask[2];
      if constexpr (decltype(masked)::value) {
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          vmask[tau][0] = (kvalid[tau * 4 + 0] ? 0x0000FFFFu : 0u) | (kvalid[tau * 4 + 1] ? 0xFFFF0000u : 0u);
          vmask[tau][1] = (kvalid[tau * 4 + 2] ? 0x0000FFFFu : 0u) | (kvalid[tau * 4 + 3] ? 0xFFFF0000u : 0u);
        }
      }
      auto vop = [&](int dt) {
        u32x2 va[2];
#pragma unroll
        for (int tau = 0; tau < 2; ++tau) {
          if constexpr (U8) {
            va[tau] = u8x4_to_16<QT>(r.v[tau][dt / 4][dt % 4]);
          } else {
            const u32x4 w = r.v[tau][dt / 2];
            va[tau] = (dt % 2) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]};
            if constexpr (decltype(masked)::value) va[tau] &= vmask[tau];
          }
        }
        return u32x4{va[0][0], va[0][1], va[1][0], va[1][1]};
      };
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x4 va = vop(dt);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][dt] = mfma32<QT>(va, pb_hi[rb], o[rb][dt]);
      }
      if constexpr (QT == kBF16) {
        // all hi products, then all lo: consecutive MFMAs never update the
        // same accumulator
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x4 va = vop(dt);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[rb][dt] = mfma32<QT>(va, pb_lo[rb], o[rb][dt]);
        }
      }
    };
    if (U8 || interior)
      pv(std::false_type{});
    else
      pv(std::true_type{});
  };

  // -------------------------------------------------------------------------
  // Half-step path (HR > 0, 16-slot pages): the wavefront's share of the
  // segment is taken one sub-tile (16 keys) at a time through a ring of HR
  // register sets, and
  // the loads of half-step j + HR are issued as soon as half-step j has been
  // computed, so loads stay in flight while the wavefront computes.  Half-
  // steps past the wavefront's last are still issued (the count of
  // outstanding loads stays static, so the compiler's waits are exact) but
  // every lane of them reads the same 16 bytes of the segment's first page:
  // one cache line, no bandwidth.  PV runs as 16x16x16 products over the
  // sub-tile's 16 keys.
  // -------------------------------------------------------------------------
  struct Half {
    u32x4 k[LK];
    u32x4 v[LV];
    u32x4 ks, vs;
  };
  auto load_half = [&](int st, int tau, Half& r, bool real, bool with_q) {
    size_t row0;
    int lane_off;
    if (real) {
      row0 = tile_of(st, tau);
      lane_off = lane * 16;
    } else {
      row0 = ((size_t)s_bt[0] * Hkv + h) * BS;           // a valid page; one line for all lanes
      lane_off = 0;
    }
    const char* kp = kb + row0 * D * EB + lane_off;
#pragma unroll
    for (int c = 0; c < LK; ++c) r.k[c] = ld16_stream(kp + (real ? c * 1024 : 0));
    if (with_q) load_q();
    const char* vp = vb + row0 * D * EB + lane_off;
#pragma unroll
    for (int c = 0; c < LV; ++c) r.v[c] = ld16_stream(vp + (real ? c * 1024 : 0));
    if constexpr (U8) {
      const size_t srow = (row0 + (real ? q4 * 4 : 0)) * 4;
      r.ks = ld16_stream(kszb + srow);
      r.vs = ld16_stream(vszb + srow);
    }
  };

  auto compute_half = [&](int st, int tau, Half& r) {
    const int key0 = si.base + st * kKeysPerStep + tau * 16;
    // S^T for the sub-tile: lane (row, q4) gets keys key0 + 4*q4 + 0..3
    float sv[RB][4];
    {
      f32x4 acc0[RB], acc1[RB];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) acc0[rb] = acc1[rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if constexpr (U8) {
#pragma unroll
        for (int c2 = 0; c2 < LK; ++c2) {
          const u32x4 w = r.k[c2];
          const u32x2 a0 = u8x4_to_16<QT>(w[0]), a1 = u8x4_to_16<QT>(w[1]);
          const u32x2 a2 = u8x4_to_16<QT>(w[2]), a3 = u8x4_to_16<QT>(w[3]);
          const u32x4 k0 = {a0[0], a0[1], a1[0], a1[1]}, k1 = {a2[0], a2[1], a3[0], a3[1]};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc0[rb] = mfma32<QT>(k0, qreg[rb][2 * c2], acc0[rb]);
            acc1[rb] = mfma32<QT>(k1, qreg[rb][2 * c2 + 1], acc1[rb]);
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const f32x4 acc = acc0[rb] + acc1[rb];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float sk = lo_f16(r.ks[e]), zk = hi_f16(r.ks[e]) + kU8Bias<QT>;
            sv[rb][e] = sk * (acc[e] - zk * qsum[rb]) * a.scale_log2;
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < QC; c += 2) {
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) {
            acc0[rb] = mfma32<QT>(r.k[c], qreg[rb][c], acc0[rb]);
            if (c + 1 < QC) acc1[rb] = mfma32<QT>(r.k[c + 1], qreg[rb][c + 1], acc1[rb]);
          }
        }
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const f32x4 acc = acc0[rb] + acc1[rb];
#pragma unroll
          for (int e = 0; e < 4; ++e) sv[rb][e] = acc[e] * a.scale_log2;
        }
      }
    }
    const bool interior = key0 >= lo_max && key0 + 16 <= all_see;
    bool kvalid[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) kvalid[e] = true;
    if (!interior) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = key0 + q4 * 4 + e;
        kvalid[e] = t >= si.lo0 && t < si.ctx;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) {
          const bool seen = t >= lo_r[rb] && (t < si.L || (t < si.ctx && ((vis_r[rb] >> (t - si.L)) & 1u)));
          sv[rb][e] = seen ? sv[rb][e] : -INFINITY;
        }
      }
    }
    u32x2 pb_hi[RB], pb_lo[RB];
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      float mx = fmaxf(fmaxf(sv[rb][0], sv[rb][1]), fmaxf(sv[rb][2], sv[rb][3]));
      mx = group_max(mx);
      const bool need = mx > m_run[rb] + kRescaleLog2;
      if (__any(need)) {
        const float m_new = need ? mx : m_run[rb];
        const float alpha = __builtin_amdgcn_exp2f(m_run[rb] - (m_new == -INFINITY ? 0.f : m_new));
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) o[rb][dt] *= alpha;
        l_run[rb] *= alpha;
        c_run[rb] *= alpha;
        m_run[rb] = m_new;
      }
      const float m_use = m_run[rb] == -INFINITY ? 0.f : m_run[rb];
      float p[4];
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = __builtin_amdgcn_exp2f(sv[rb][e] - m_use);
        psum += p[e];
      }
      l_run[rb] += psum;
      if constexpr (U8) {
        float csum = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t w = r.vs[e];
          float sp = kvalid[e] ? p[e] * lo_f16(w) : 0.f;
          if constexpr (QT == kF16) sp = (float)(_Float16)sp;
          csum += kvalid[e] ? sp * (hi_f16(w) + kU8Bias<QT>) : 0.f;
          p[e] = sp;
        }
        c_run[rb] += csum;
      }
      pack_p4<QT>(p, pb_hi[rb], pb_lo[rb]);
    }
    // PV over the sub-tile's 16 keys: A of lane (d, q4) is V of keys
    // 4*q4 + 0..3 at d, B the lane's four weights
    auto pv = [&](auto masked) {
      u32x2 vmask;
      if constexpr (decltype(masked)::value) {
        vmask[0] = (kvalid[0] ? 0x0000FFFFu : 0u) | (kvalid[1] ? 0xFFFF0000u : 0u);
        vmask[1] = (kvalid[2] ? 0x0000FFFFu : 0u) | (kvalid[3] ? 0xFFFF0000u : 0u);
      }
      auto vop = [&](int dt) {
        u32x2 va;
        if constexpr (U8) {
          va = u8x4_to_16<QT>(r.v[dt / 4][dt % 4]);
        } else {
          const u32x4 w = r.v[dt / 2];
          va = (dt % 2) ? u32x2{w[2], w[3]} : u32x2{w[0], w[1]};
          if constexpr (decltype(masked)::value) va &= vmask;
        }
        return va;
      };
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u32x2 va = vop(dt);
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) o[rb][dt] = mfma16<QT>(va, pb_hi[rb], o[rb][dt]);
      }
      if constexpr (QT == kBF16) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const u32x2 va = vop(dt);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[rb][dt] = mfma16<QT>(va, pb_lo[rb], o[rb][dt]);
        }
      }
    };
    if (U8 || interior)
      pv(std::false_type{});
    else
      pv(std::true_type{});
  };

  if constexpr (HR > 0 && BS >= 16) {
    // The segment's half-steps k = 0 .. 2 (st_end - st_begin) - 1 (sub-tile
    // k % 2 of step st_begin + k / 2) go to the wavefronts round-robin: this
    // one's j-th is k = wave + j NW.  A segment one step longer than a
    // multiple of NW (the T new keys past a round context) then gives that
    // step's halves to two wavefronts instead of a whole step to one.
    const int nseg = 2 * max(st_end - st_begin, 0);
    const int nh = wave < nseg ? (nseg - 1 - wave) / NW + 1 : 0;
    auto hst = [&](int j) { return st_begin + ((wave + j * NW) >> 1); };
    auto htau = [&](int j) { return (wave + j * NW) & 1; };
    if (nh > 0) {
      Half ring[HR];
#pragma unroll
      for (int i = 0; i < HR; ++i) load_half(hst(i), htau(i), ring[i], i < nh, i == 0);
      finish_q();
      for (int j0 = 0; j0 < nh; j0 += HR) {
#pragma unroll
        for (int i = 0; i < HR; ++i) {
          const int j = j0 + i;
          if (j < nh) compute_half(hst(j), htau(j), ring[i]);
          const int jn = j + HR;
          load_half(hst(jn), htau(jn), ring[i], jn < nh, false);
        }
      }
    }
  } else {
    // Steps st_begin + wave, + NW, ...: one register set; the other
    // wavefronts of the CU keep the memory system busy while this one computes.
    Step ra;
    int st = st_begin + wave;
    if (st < st_end) {
      load_step(st, ra, true);
      finish_q();
      compute_step(st, ra);
      for (st += NW; st < st_end; st += NW) {
        load_step(st, ra, false);
        compute_step(st, ra);
      }
    }
  }

  // the merge buffer reuses the staging area: every wavefront is done with it
  if constexpr (ALIAS) __syncthreads();

  // Row sums: each lane group holds a quarter of the keys.  Then merge the
  // wavefronts of the workgroup: M = max_w m_w, then sum the partials
  // rescaled by 2^(m_w - M), in a fixed order (bitwise repeatable).
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l_run[rb] = group_sum(l_run[rb]);
    const int r = rb * kRows + n16;
    if constexpr (U8) {
      c_run[rb] = group_sum(c_run[rb]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) o[rb][dt] -= c_run[rb];
      // f16 q: a weight (at most 2^kRescaleLog2 against the reference max)
      // times a V scale above 65504 / 256 can round to inf in f16; the row
      // sum of those products is then inf or NaN for good.  Never silent:
      // the workgroup's partials become NaN and the status word is set.
      if constexpr (QT == kF16)
        if (r < R && !__builtin_isfinite(c_run[rb])) s_bad = 1;
    }
    if (q4 == 0) {
      s_m[wave][r] = m_run[rb];
      s_l[wave][r] = l_run[rb];
    }
    if (r < R) {                                              // padding rows are never read
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<f32x4*>(&s_o[wave][r][dt * 16 + q4 * 4]) = o[rb][dt];
    }
  }
  __syncthreads();

  const bool bad = s_bad != 0;
  constexpr int V4 = D / 4;                                   // float4 columns per row
  for (int x = threadIdx.x; x < R * V4; x += NW * kWave) {
    const int r = x / V4;
    const int c4 = (x % V4) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, s_m[w][r]);
    const int rt = si.b0 + r % T;
    const int rh = h * a.G + r / T;
    const size_t row = ((size_t)rt * a.Hq + rh) * a.S + j;   // partials are per token
    if (a.direct) {
      // the one segment: the normalised row (NaN for a row with no key,
      // 0 / 0, as the combine would make it)
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      float lsum = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float f = __builtin_amdgcn_exp2f(s_m[w][r] - M);
          acc += f * *reinterpret_cast<const f32x4*>(&s_o[w][r][c4]);
          lsum += f * s_l[w][r];
        }
      }
      u32x2 packed;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const float x0 = bad ? NAN : acc[2 * e] / lsum, x1 = bad ? NAN : acc[2 * e + 1] / lsum;
        if constexpr (QT == kF16) {
          packed[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x0) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x1) << 16);
        } else {
          packed[e] = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x0) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)x1) << 16);
        }
      }
      uint16_t* dst = reinterpret_cast<uint16_t*>(a.out) + ((size_t)rt * a.Hq + rh) * D + c4;
      *reinterpret_cast<u32x2*>(dst) = packed;
      continue;
    }
    if (M == -INFINITY) {                                     // no key of this row here
      if (c4 == 0) {
        a.ws_ml[row * 2 + 0] = bad ? NAN : -INFINITY;
        a.ws_ml[row * 2 + 1] = 0.f;
      }
      continue;
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float lsum = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = __builtin_amdgcn_exp2f(s_m[w][r] - M);
      acc += f * *reinterpret_cast<const f32x4*>(&s_o[w][r][c4]);
      lsum += f * s_l[w][r];
    }
    // plain stores: the combine reads the partials right after this kernel
    // (measured 0.1-0.9 us per call faster than nontemporal stores)
    *reinterpret_cast<f32x4*>(&a.ws_o[row * D + c4]) = acc;
    if (c4 == 0) {
      a.ws_ml[row * 2 + 0] = bad ? NAN : M;
      a.ws_ml[row * 2 + 1] = lsum;
    }
  }
  if (bad && threadIdx.x == 0) atomicExch(a.status, kDeviceContract);
}

// ---------------------------------------------------------------------------
// Launchers: one instance per (q dtype, cache dtype, D, block size, row
// blocks); each pa_segment_*.hip instantiates one cache dtype.
// ---------------------------------------------------------------------------
template <int QT, int KV, int D, int BS, int RB, int PL, int SMALL = 0>
hipError_t launch_seg(const SegmentArgs& a, dim3 grid, hipStream_t st, hipEvent_t ev0, hipEvent_t ev1) {
  constexpr SegConfig c = SMALL ? seg_config_small(KV, D, BS, SMALL) : seg_config(KV, D, RB, BS, PL);
  static_assert(c.waves_per_group <= 4 * c.waves_per_simd, "a workgroup must fit on one CU");
  // the half-step path reads tiled pages only
  constexpr int HR = PL == kPagesTiled ? c.half_ring : 0;
  constexpr auto kern = pa_segment<QT, KV, D, BS, c.waves_per_group, c.waves_per_simd, RB, HR, PL>;
  return launch_kernel(reinterpret_cast<const void*>(kern), grid, dim3(c.waves_per_group * kWave),
                       st, a, ev0, ev1);
}

template <int QT, int KV, int D, int BS, int PL>
hipError_t dispatch_rb(const SegmentArgs& a, int rb, dim3 grid, hipStream_t st, hipEvent_t e0,
                       hipEvent_t e1) {
  switch (rb) {
    case 1:
      if constexpr (BS >= 16 && PL == kPagesTiled) {
        if (a.small_groups == 2) return launch_seg<QT, KV, D, BS, 1, PL, 2>(a, grid, st, e0, e1);
        if (a.small_groups == 4) return launch_seg<QT, KV, D, BS, 1, PL, 4>(a, grid, st, e0, e1);
      }
      return launch_seg<QT, KV, D, BS, 1, PL>(a, grid, st, e0, e1);
    case 2:
      if constexpr (BS >= 16 && max_row_blocks(KV, D) >= 2) return launch_seg<QT, KV, D, BS, 2, PL>(a, grid, st, e0, e1);
      break;
    case 3:
      if constexpr (BS >= 16 && max_row_blocks(KV, D) >= 3) return launch_seg<QT, KV, D, BS, 3, PL>(a, grid, st, e0, e1);
      break;
    case 4:
      if constexpr (BS >= 16 && max_row_blocks(KV, D) >= 4) return launch_seg<QT, KV, D, BS, 4, PL>(a, grid, st, e0, e1);
      break;
  }
  return hipErrorInvalidValue;
}

template <int QT, int KV, int D, int PL>
hipError_t dispatch_bs(const SegmentArgs& a, int bs, int rb, dim3 grid, hipStream_t st,
                       hipEvent_t e0, hipEvent_t e1) {
  switch (bs) {
    case 1:
      // a 1-slot page is the same in both layouts
      return dispatch_rb<QT, KV, D, 1, kPagesTiled>(a, rb, grid, st, e0, e1);
    case 2: return dispatch_rb<QT, KV, D, 2, PL>(a, rb, grid, st, e0, e1);
    case 4: return dispatch_rb<QT, KV, D, 4, PL>(a, rb, grid, st, e0, e1);
    case 8: return dispatch_rb<QT, KV, D, 8, PL>(a, rb, grid, st, e0, e1);
    case 16: return dispatch_rb<QT, KV, D, 16, PL>(a, rb, grid, st, e0, e1);
    case 32: return dispatch_rb<QT, KV, D, 32, PL>(a, rb, grid, st, e0, e1);
    case 64: return dispatch_rb<QT, KV, D, 64, PL>(a, rb, grid, st, e0, e1);
  }
  return hipErrorInvalidValue;
}

template <int QT, int KV, int PL>
hipError_t dispatch_d_pl(const SegmentArgs& a, int D, int bs, int rb, dim3 grid, hipStream_t st,
                         hipEvent_t e0, hipEvent_t e1) {
  switch (D) {
    case 64: return dispatch_bs<QT, KV, 64, PL>(a, bs, rb, grid, st, e0, e1);
    case 128: return dispatch_bs<QT, KV, 128, PL>(a, bs, rb, grid, st, e0, e1);
    case 256: return dispatch_bs<QT, KV, 256, PL>(a, bs, rb, grid, st, e0, e1);
  }
  return hipErrorInvalidValue;
}

template <int QT, int KV>
hipError_t dispatch_d(const SegmentArgs& a, int D, int bs, int rb, dim3 grid, hipStream_t st,
                      hipEvent_t e0, hipEvent_t e1) {
  if (a.page_layout == kPagesRowMajor)
    return dispatch_d_pl<QT, KV, kPagesRowMajor>(a, D, bs, rb, grid, st, e0, e1);
  return dispatch_d_pl<QT, KV, kPagesTiled>(a, D, bs, rb, grid, st, e0, e1);
}

}  // namespace pav
