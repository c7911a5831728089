// pa_kernels.h — what the host side of libpa_verify passes to the gfx950
// kernels (internal; not part of the C ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pav {

enum : int { kF16 = 0, kBF16 = 1, kU8 = 2 };
enum : int { kPagesTiled = 0, kPagesRowMajor = 1 };   // values of pa_page_layout

constexpr int kKeysPerStep = 32;     // keys one wavefront consumes per iteration
constexpr int kRows = 16;            // stacked query rows per MFMA tile (one row block)
constexpr int kMaxT = 16;            // verify rows per sequence (tree-mask words are 16 bits used)
constexpr int kWavesPerGroup = 4;    // wavefronts per segment workgroup (default of the table below)
// LDS slots for a segment's block ids: 1040, or 2080 for 1-slot pages (one id
// per key), whose segments would otherwise span at most 32 steps.
constexpr int seg_block_slots(int bs) { return bs == 1 ? 2080 : 1040; }
constexpr int kDeviceContract = 5;   // value of PA_ERR_DEVICE_CONTRACT
constexpr float kRescaleLog2 = 8.f;  // softmax reference max moves only past this margin
#ifndef PA_HALF_RING_U8
#define PA_HALF_RING_U8 2
#endif
constexpr int kHalfRingU8 = PA_HALF_RING_U8;   // register sets of the u8 head_dim-256 half-step path

struct SegmentArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* ksz;                   // u8 only: f16 (scale, zero point) per token
  const void* vsz;
  const int32_t* bt;
  const int32_t* past_lens;
  const int32_t* sb;
  const uint32_t* tree;              // optional [num_tokens] tree-mask words; null = causal rows
  float* ws_o;                       // [num_tokens, Hq, S, D] unnormalised partial outputs
  float* ws_ml;                      // [num_tokens, Hq, S, 2] (max in log2 units, sum)
  int32_t* status;                   // sticky device status word
  // [sb_words] one word per wavefront of segment workgroup 0, nonzero when
  // subsequence_begins breaks its contract (read by the combine kernel)
  int32_t* sb_check;
  int32_t sb_words;
  int32_t num_seqs, num_tokens, Hq, Hkv, G;
  int32_t num_blocks, mbps, window, max_ctx;
  int32_t max_q;                     // bound on T_s the host planned for (<= kMaxT)
  int32_t S, steps_per_seg, n_steps;   // segments; max steps of one segment; steps the host plans for
  int32_t worklist;                  // ragged batch: chunks of device-chosen size, see below
  int32_t target_items;              // work-list chunks per KV head the chunk size aims at
  int32_t max_sps;                   // most steps whose block ids fit the LDS table
  float scale_log2;                  // scale * log2(e)
  int32_t page_layout;               // kPagesTiled or kPagesRowMajor
  // S == 1: the segment kernel normalises its rows and writes them to out
  // ([num_tokens, Hq, D] in the q dtype) instead of partials
  int32_t direct;
  void* out;
  int32_t small_groups;              // host dispatch only: 0, or the waves of the small-workgroup instance
};

struct AppendArgs {
  const void* k_new;                 // [num_tokens, Hkv, D] in the q dtype
  const void* v_new;
  void* k_cache;
  void* v_cache;
  void* ksz;                         // u8 only: f16 (scale, zero point) per token
  void* vsz;
  const int32_t* bt;
  const int32_t* past_lens;
  const int32_t* sb;
  int32_t* status;                   // sticky device status word
  int32_t num_seqs, num_tokens, Hkv, bs, mbps, num_blocks, max_q;
  int32_t page_layout;               // kPagesTiled or kPagesRowMajor
};

struct CombineArgs {
  SegmentArgs seg;
  void* out;
  int32_t num_tokens, Hq;
  // > 1 (gcd of the device's XCD count and Hkv): workgroup i takes a
  // (token, q head) pair whose KV head is congruent to i modulo xcds.
  // Workgroups go to the XCDs round-robin by linear id, so it runs on an XCD
  // whose L2 may still hold that KV head's partials from the segment kernel
  // (all of them when the XCD count divides Hkv).
  int32_t xcds;
  int32_t head_dim;
};

// ev0/ev1: optional events timestamped by the segment kernel's own dispatch
// rb: 16-row blocks of stacked query rows (1 to max_row_blocks).
// One function per cache dtype, each in its own translation unit.
hipError_t launch_segment_f16(const SegmentArgs& a, int D, int bs, int rb, dim3 grid,
                              hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_segment_bf16(const SegmentArgs& a, int D, int bs, int rb, dim3 grid,
                               hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_segment_u8(const SegmentArgs& a, int q_dtype, int D, int bs, int rb, dim3 grid,
                             hipStream_t st, hipEvent_t ev0, hipEvent_t ev1);
hipError_t launch_combine(const CombineArgs& a, int out_dtype, int D, int threads, dim3 grid,
                          hipStream_t st);
// After a direct segment kernel: turns every output row into NaN and sets
// the status when the segment kernel found subsequence_begins broken.
hipError_t launch_finish(const CombineArgs& a, int out_dtype, int threads, dim3 grid, hipStream_t st);
hipError_t launch_append(const AppendArgs& a, int q_dtype, int kv_dtype, int D, hipStream_t st);
// Most steps a segment or work-list chunk may span: its block ids (one more
// for a step that starts inside a page, one more for the last page) must fit
// the seg_block_slots(bs)-entry LDS table.
constexpr int max_steps_per_segment(int bs) { return (seg_block_slots(bs) - 2) * bs / kKeysPerStep; }

// Work-list batches hold 2 .. kWlSeqs sequences: every wavefront keeps their
// metadata in registers, kWlCached lane-strided groups of 64.
constexpr int kWlCached = 4;
constexpr int kWlSeqs = kWlCached * 64;
// the work list's exact float ceiling division needs chunk sizes below 2^16
static_assert(max_steps_per_segment(64) < 65536, "chunk sizes must stay below 2^16");

// Combine grid: one 64-thread workgroup per (token, q head) row and 64-column
// slice of it (same-box A/B, us per call: see the combine kernel).
constexpr int combine_slices(int D) { return D / 64; }
// The check kernel of direct calls: one 256-thread workgroup per CU.
constexpr int kFinishGroups = 256;
constexpr int kFinishThreads = 256;

// Per (cache dtype, head_dim, row blocks, block size): wavefronts per SIMD
// the segment kernel is compiled for (its register budget, no spills; each
// wavefront holds one step in registers: load, then compute), the segment
// workgroups the planner puts on each CU (at most the resident count, 4
// SIMDs per CU) and the wavefronts per workgroup.  Measured on MI355X at 32k
// context:
// head_dim 128 (16-bit) and u8 head_dim 256 run best as one 8-wavefront
// workgroup per CU, two wavefronts per SIMD with one step each (32 q / 8 KV
// heads, T = 3: 27.6 vs 28.2 µs per call for 4 wavefronts with two steps each; u8 21.4 vs
// 22.5 µs) — two workgroups of 4 instead would double the partials the
// combine reads.  The same holds elsewhere (32 q / 8 KV heads, T = 3, at
// 32k, µs per call): head_dim 64 as two 8-wavefront workgroups per CU at four
// wavefronts per SIMD, 17.4 vs 17.7 for four 4-wavefront ones (one
// 16-wavefront one: 18.6); u8 head_dim 128 (16 q / 4 KV heads) as one
// 8-wavefront workgroup at two per SIMD, 14.5 vs 15.4 for one 4-wavefront
// workgroup with two steps in flight (12 wavefronts at three per SIMD:
// 15.2).  Two row blocks at head_dim <= 128 still fit two
// wavefronts per SIMD (T = 5 and 8 at 32k: 30.0 and 30.7 us per call against
// 30.35 and 31.3 at one), and so do three or four at head_dim 64 (32 q / 8
// KV heads, T = 12 and 16 at 32k: 21.7 and 25.0 us per call against 25.2
// and 28.6 at one); more row blocks at head_dim 128, or head_dim 256, need the whole
// register file of one wavefront per SIMD (and the LDS merge buffer allows
// one workgroup per CU).
struct SegConfig {
  int waves_per_simd;
  int groups_per_cu;
  int waves_per_group = kWavesPerGroup;
  int half_ring = 0;   // > 0: half-step path with this many register sets (16-slot pages)
};
// The half-step path (two register sets of one 16-slot sub-tile each, see the
// segment kernel) is used where it measured faster, same-box A/B of graph-
// replayed us per call: u8 head_dim 256, 21.08 -> 20.76 (three sets 21.99);
// 16-bit head_dim 128, ragged batch 64.19 -> 63.85, 32k 26.20 -> 26.13.  Not
// at 16-bit head_dim 256 (window layer 8.63 -> 10.12, global 83.98 -> 84.69)
// or head_dim 64 (16.54 -> 17.05).
constexpr SegConfig seg_config_tiled(int kv_dtype, int D, int rb, int bs) {
  // Pages of fewer than 16 slots: one 8-wavefront workgroup per CU as for
  // 16-slot pages (32 q / 8 KV heads, head_dim 128, T = 3 at 32k, us per
  // call: 2 slots 29.8 vs 29.9 for two
  // 4-wavefront groups, 4 slots 27.6 vs 28.1, 8 slots 27.8 vs 28.0).
  if (bs < 16) return D >= 256 ? SegConfig{1, 1} : SegConfig{2, 1, 8};
  if (rb > 1) return (rb == 2 && D <= 128) || D <= 64 ? SegConfig{2, 1, 8} : SegConfig{1, 1};
  if (kv_dtype == kU8)
    return D >= 256 ? SegConfig{2, 1, 8, kHalfRingU8} : D >= 128 ? SegConfig{2, 1, 8} : SegConfig{4, 4};
  return D >= 256 ? SegConfig{1, 1} : D >= 128 ? SegConfig{2, 1, 8, 2} : SegConfig{4, 2, 8};
}
// One-segment calls over short contexts (every workgroup one short
// sequence, most of an 8-wavefront workgroup idle): workgroups of 2 or 4
// wavefronts at the same wavefronts per SIMD, so more of them are in
// flight per CU.  One row block, tiled pages of 16 or more slots.  Same-box
// A/B, graph-replayed us per call, 4096 sequences of 16..256 keys (at most
// 9 steps) / 512 of 64..1024 (33 steps): 8 wavefronts 652 / 157.6, four 365
// / 129.7, two 331 / 136.3, one 330 / 143.8.  Two up to kSmallSplitSteps
// steps, four up to kSmallMaxSteps.
constexpr int kSmallSplitSteps = 16;
constexpr int kSmallMaxSteps = 48;
constexpr int small_waves(int n_steps) {
  return n_steps <= kSmallSplitSteps ? 2 : n_steps <= kSmallMaxSteps ? 4 : 0;
}
// Row-major pages stage every step through LDS on the full-step path; at
// u8 head_dim 256 that path at two wavefronts per SIMD spills 368-484 B per
// lane, so there it runs one wavefront per SIMD with the whole register file.
constexpr SegConfig seg_config(int kv_dtype, int D, int rb, int bs = 16, int pl = kPagesTiled) {
  return pl == kPagesRowMajor && kv_dtype == kU8 && D >= 256 && bs >= 16 ? SegConfig{1, 1}
                                                                         : seg_config_tiled(kv_dtype, D, rb, bs);
}
constexpr SegConfig seg_config_small(int kv_dtype, int D, int bs, int nw) {
  const SegConfig c = seg_config(kv_dtype, D, 1, bs);
  return SegConfig{c.waves_per_simd, 4 * c.waves_per_simd / nw, nw, c.half_ring};
}
constexpr int groups_per_cu(int kv_dtype, int D, int rb, int bs, int pl = kPagesTiled) {
  return seg_config(kv_dtype, D, rb, bs, pl).groups_per_cu;
}
// Row blocks built per (cache dtype, head_dim): each adds D/4 accumulator
// and D/8 query registers per lane and 16 * (D + 4) * 16 B of LDS; these are
// the largest counts that compile without register spills.
constexpr int max_row_blocks(int kv_dtype, int D) {
  return D <= 64 ? 4 : D <= 128 ? 3 : kv_dtype == kU8 ? 2 : 1;
}
// Pages of fewer than 16 slots are built for one row block only.
constexpr int max_row_blocks(int kv_dtype, int D, int bs) {
  return bs < 16 ? 1 : max_row_blocks(kv_dtype, D);
}
static_assert(kWavesPerGroup == 4, "the table above assumes 4-wavefront workgroups");

}  // namespace pav
