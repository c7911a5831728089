// pa_verify.hip — host side of libpa_verify.so: argument validation, the
// launch planner and the C ABI declared in include/pa_verify.h.
//
// Nothing here touches the device before the arguments have been checked,
// so every host-side error path runs without a GPU.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <mutex>
#include <set>
#include <tuple>

#include "pa_kernels.h"
#include "pa_verify.h"

namespace {

using pav::kKeysPerStep;

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Upper bound on segment-kernel workgroups per resident slot (see make_plan).
constexpr int64_t kMaxRounds = 8;
// T_s bound when the caller gives none (max_query_len == 0).
constexpr int64_t kDefaultQueryLen = 4;

bool aligned(const void* x, uintptr_t a) { return (reinterpret_cast<uintptr_t>(x) & (a - 1)) == 0; }

bool is_pow2_in(int v, int lo, int hi) {
  if (v < lo || v > hi) return false;
  return (v & (v - 1)) == 0;
}

// Bound on the new tokens of one sequence: max_query_len when given, else
// the classic verify bound of 4 (or fewer when num_tokens and num_seqs
// allow no more).
int64_t query_bound(const pa_verify_params* p) {
  const int64_t t = p->max_query_len > 0 ? p->max_query_len
                                         : std::min<int64_t>(kDefaultQueryLen, (int64_t)p->num_tokens - p->num_seqs + 1);
  return std::max<int64_t>(1, std::min<int64_t>(t, pav::kMaxT));
}

// Host-checkable contract.  u8_entry selects which entry point is asking.
int validate(const pa_verify_params* p, int32_t max_ctx, bool u8_entry) {
  if (!p) return PA_ERR_INVALID_ARG;
  if (p->num_seqs < 1 || p->num_tokens < p->num_seqs || p->num_q_heads < 1 ||
      p->num_kv_heads < 1 || p->head_dim < 1 || p->block_size < 1 || p->num_blocks < 1 ||
      p->max_blocks_per_seq < 1 || p->sliding_window < 0 || p->num_segments < 0 || max_ctx < 1)
    return PA_ERR_INVALID_ARG;
  if (p->num_q_heads % p->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (cdiv(max_ctx, p->block_size) > p->max_blocks_per_seq) return PA_ERR_INVALID_ARG;
  const int G = p->num_q_heads / p->num_kv_heads;
  if (!is_pow2_in(G, 1, 8)) return PA_ERR_UNSUPPORTED;
  if (p->head_dim != 64 && p->head_dim != 128 && p->head_dim != 256) return PA_ERR_UNSUPPORTED;
  if (p->block_size != 1 && p->block_size != 2 && p->block_size != 4 && p->block_size != 8 &&
      p->block_size != 16 && p->block_size != 32 && p->block_size != 64)
    return PA_ERR_UNSUPPORTED;
  if (p->q_dtype != PA_F16 && p->q_dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  if (u8_entry) {
    if (p->kv_dtype != PA_U8) return PA_ERR_UNSUPPORTED;
  } else {
    if (p->kv_dtype != p->q_dtype) return PA_ERR_UNSUPPORTED;
  }
  // sizes that index 32-bit device arithmetic stay in range
  if ((int64_t)p->num_blocks * p->num_kv_heads * p->block_size > INT32_MAX) return PA_ERR_UNSUPPORTED;
  if ((int64_t)p->num_tokens * p->num_q_heads > INT32_MAX / 4) return PA_ERR_UNSUPPORTED;
  // the combine launches one thread per output element
  if ((int64_t)p->num_tokens * p->num_q_heads * p->head_dim > UINT32_MAX) return PA_ERR_UNSUPPORTED;
  if (p->num_seqs > 65535 || p->num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;   // grid y, x limits
  if (p->max_query_len < 0) return PA_ERR_INVALID_ARG;
  if (p->max_query_len > pav::kMaxT) return PA_ERR_UNSUPPORTED;
  if ((int64_t)G * query_bound(p) >
      (int64_t)pav::kRows * pav::max_row_blocks(p->kv_dtype, p->head_dim, p->block_size))
    return PA_ERR_UNSUPPORTED;
  if (p->tree_mask && p->sliding_window > 0) return PA_ERR_UNSUPPORTED;
  if (p->page_layout != PA_PAGES_TILED && p->page_layout != PA_PAGES_ROW_MAJOR) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// 16-row blocks of the segment kernel for these params: enough for
// G * (bound on T_s) stacked rows.
int row_blocks(const pa_verify_params* p) {
  const int64_t rows = (int64_t)(p->num_q_heads / p->num_kv_heads) * query_bound(p);
  return (int)std::max<int64_t>(1, cdiv(rows, pav::kRows));
}

int make_plan(const pa_verify_params* p, int32_t max_ctx, int32_t num_cus, pa_verify_plan* pl) {
  const int bs = p->block_size;
  int64_t span = max_ctx;
  if (p->sliding_window > 0) {
    // rows of one sequence read at most W + T - 1 keys; the first step is
    // aligned down to a step boundary
    span = std::min<int64_t>(span, (int64_t)p->sliding_window + query_bound(p) - 1 + kKeysPerStep - 1);
  }
  const int64_t n_steps = cdiv(span, kKeysPerStep);
  // a segment's block ids must fit the kernel's LDS staging buffer
  const int64_t max_sps = pav::max_steps_per_segment(bs);
  int64_t S;
  if (p->num_segments > 0) {
    S = p->num_segments;
  } else {
    // Enough segments that one sequence of max_context_len keys alone
    // covers every resident workgroup slot of the GPU (every CU busy at
    // batch 1, and in a ragged batch the longest sequence is not left to a
    // few CUs), but at most kMaxRounds rounds of workgroups in all.
    const int64_t groups =
        (int64_t)num_cus * pav::groups_per_cu(p->kv_dtype, p->head_dim, row_blocks(p), p->block_size,
                                              p->page_layout);
    const int64_t pairs = (int64_t)p->num_kv_heads * p->num_seqs;
    S = cdiv(groups, p->num_kv_heads);
    S = std::min(S, std::max<int64_t>(cdiv(groups, pairs), kMaxRounds * groups / pairs));
  }
  S = std::max<int64_t>(std::min(S, n_steps), cdiv(n_steps, max_sps));
  if (S > 65535) return PA_ERR_UNSUPPORTED;           // grid z limit
  const int64_t sps = cdiv(n_steps, S);               // longest segment; the others are >= sps - 1
  pl->num_segments = (int32_t)S;
  pl->steps_per_segment = (int32_t)sps;
  pl->num_steps = (int32_t)n_steps;
  pl->row_blocks = row_blocks(p);
  pl->keys_per_step = kKeysPerStep;
  pl->span = (int32_t)span;
  const int nw = pav::seg_config(p->kv_dtype, p->head_dim, pl->row_blocks, p->block_size, p->page_layout)
                     .waves_per_group;
  pl->waves_per_group = nw;
  pl->max_steps_per_segment = (int32_t)max_sps;
  pl->grid[0] = p->num_kv_heads;
  pl->grid[1] = p->num_seqs;
  pl->grid[2] = (int32_t)S;
  pl->target_items = (int32_t)std::max<int64_t>(
      1, cdiv((int64_t)num_cus * pav::groups_per_cu(p->kv_dtype, p->head_dim, pl->row_blocks,
                                                    p->block_size, p->page_layout), p->num_kv_heads));
  // The work list pays where a few sequences of unequal length must share
  // the GPU.  Every sequence has at least one chunk, so with more sequences
  // than target_items the device's chunk size would be the longest
  // sequence's (capped by the LDS table): chunks the same as the fixed
  // per-sequence segments up to their cut points, at the cost of a scan
  // over the batch in every workgroup.  Those batches, and any of more than
  // kWlSeqs sequences, take the fixed segments.
  pl->worklist = p->num_seqs > 1 && p->num_seqs <= std::min<int64_t>(pl->target_items, pav::kWlSeqs);
  if (pl->worklist) {
    // a ragged batch: one workgroup per work-list chunk, at most
    // max(target, every sequence at its fewest chunks); past the grid's z
    // limit, fixed segments instead
    const int64_t most = std::max<int64_t>(pl->target_items, (int64_t)p->num_seqs * cdiv(n_steps, max_sps));
    if (most > 65535) {
      pl->worklist = 0;
    } else {
      pl->grid[1] = 1;
      pl->grid[2] = (int32_t)most;
    }
  }
  pl->block_threads = nw * 64;
  const int64_t rows = (int64_t)p->num_tokens * p->num_q_heads;
  // One segment: nothing to combine.  The segment kernel writes the output
  // rows (no partials) and a check kernel of kFinishGroups workgroups
  // follows it in the combine's place.
  pl->direct = S == 1 ? 1 : 0;
  // one-segment calls over short contexts: the small-workgroup instance
  pl->small_groups = pl->direct && pl->row_blocks == 1 && bs >= 16 && p->page_layout == PA_PAGES_TILED
                         ? pav::small_waves((int)n_steps) : 0;
  if (pl->small_groups) {
    pl->waves_per_group = pl->small_groups;
    pl->block_threads = pl->small_groups * 64;
  }
  pl->combine_grid[0] = pl->direct ? pav::kFinishGroups : (int32_t)(rows * pav::combine_slices(p->head_dim));
  pl->combine_grid[1] = 1;
  pl->combine_grid[2] = 1;
  pl->combine_threads = pl->direct ? pav::kFinishThreads : 64;
  const size_t ml_bytes = pl->direct ? 0 : (size_t)rows * S * 2 * sizeof(float);
  const size_t o_bytes = pl->direct ? 0 : (size_t)rows * S * p->head_dim * sizeof(float);
  pl->workspace_bytes = 256 + ((ml_bytes + 255) / 256) * 256 + o_bytes;
  return PA_OK;
}

// Compute units of the current device, queried once per device.
int device_cus(int* cus) {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return PA_ERR_HIP;
  if (dev >= 0 && dev < 64) {
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) {
      *cus = c;
      return PA_OK;
    }
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return PA_ERR_HIP;
  if (dev >= 0 && dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  *cus = n;
  return PA_OK;
}

// XCDs of the current device (0 when the runtime cannot say), queried once
// per device.
int device_xccs() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  const int c = cache[dev].load(std::memory_order_relaxed);
  if (c != 0) return c < 0 ? 0 : c;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || n <= 0) n = -1;
  cache[dev].store(n, std::memory_order_relaxed);
  return n < 0 ? 0 : n;
}

void maybe_log(const pa_verify_params* p, const pa_verify_plan& pl, int32_t max_ctx) {
  static const bool on = [] {
    const char* e = std::getenv("PA_VERIFY_LOG");
    return e && e[0] && e[0] != '0';
  }();
  if (!on) return;
  static std::mutex mu;
  static std::set<std::tuple<int, int, int, int, int, int, int>> seen;
  std::lock_guard<std::mutex> g(mu);
  auto key = std::make_tuple(p->num_seqs, p->num_kv_heads, p->head_dim, p->block_size,
                             p->kv_dtype, pl.num_segments, pl.steps_per_segment);
  if (!seen.insert(key).second) return;
  std::fprintf(stderr,
               "[pa_verify] kv=%d D=%d bs=%d Hq=%d Hkv=%d seqs=%d max_ctx=%d W=%d -> S=%d "
               "steps/seg=%d (x%d keys) grid=(%d,%d,%d)x%d combine=%dx%d ws=%zu B\n",
               p->kv_dtype, p->head_dim, p->block_size, p->num_q_heads, p->num_kv_heads,
               p->num_seqs, max_ctx, p->sliding_window, pl.num_segments, pl.steps_per_segment,
               pl.keys_per_step, pl.grid[0], pl.grid[1], pl.grid[2], pl.block_threads,
               pl.combine_grid[0], pl.combine_threads, pl.workspace_bytes);
}

// The forward call.  Its partials and status word go to ws_base (ws_bytes):
// the caller's workspace, or for the no-allocation entry point the static
// scratch array, whose address is resolved only once the call is known to
// fit (get_scratch).
// ---------------------------------------------------------------------------
// Static scratch for pa_verify_forward_noalloc: the status word and the
// segment partials of one call, for callers that cannot allocate.  One copy
// per GPU, held until the process ends.  In host code `scratch` only names
// the symbol; its device address on the current device comes from
// hipGetSymbolAddress, once per device, and only that address is ever passed
// to a kernel.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = size_t(32) << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];                  // device address per device, once resolved

int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_HIP;
  std::lock_guard<std::mutex> g(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return PA_ERR_HIP;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return PA_OK;
}

int run(const void* q, const void* k, const void* v, const void* ksz, const void* vsz,
        const int32_t* bt, const int32_t* past_lens, const int32_t* sb, int32_t max_ctx,
        float scale, void* out, const pa_verify_params* p, bool u8_entry,
        int (*get_scratch)(void**) = nullptr) {
  int rc = validate(p, max_ctx, u8_entry);
  if (rc) return rc;
  if (!q || !k || !v || !bt || !past_lens || !sb || !out) return PA_ERR_INVALID_ARG;
  if (u8_entry && (!ksz || !vsz)) return PA_ERR_INVALID_ARG;
  // the widths the kernels access these with
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16) ||
      !aligned(bt, 4) || !aligned(past_lens, 4) || !aligned(sb, 4) || !aligned(p->tree_mask, 4))
    return PA_ERR_INVALID_ARG;
  if (u8_entry && (!aligned(ksz, 16) || !aligned(vsz, 16))) return PA_ERR_INVALID_ARG;
  if (!get_scratch && !aligned(p->workspace, 16)) return PA_ERR_WORKSPACE;
  if (!(scale == scale)) return PA_ERR_INVALID_ARG;
  int cus = 0;
  rc = device_cus(&cus);
  if (rc) return rc;
  pa_verify_plan pl;
  rc = make_plan(p, max_ctx, cus, &pl);                      // grid limits
  if (rc) return rc;
  void* ws_base = p->workspace;
  if (get_scratch) {
    if (pl.workspace_bytes > kScratchBytes) return PA_ERR_WORKSPACE;
    rc = get_scratch(&ws_base);
    if (rc) return rc;
  } else if (!p->workspace || p->workspace_bytes < pl.workspace_bytes) {
    return PA_ERR_WORKSPACE;
  }
  maybe_log(p, pl, max_ctx);

  char* ws = static_cast<char*>(ws_base);
  const size_t rows = (size_t)p->num_tokens * p->num_q_heads;
  const size_t ml_bytes = pl.direct ? 0 : ((rows * pl.num_segments * 2 * sizeof(float) + 255) / 256) * 256;
  pav::SegmentArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.ksz = ksz;
  a.vsz = vsz;
  a.bt = bt;
  a.past_lens = past_lens;
  a.sb = sb;
  a.tree = static_cast<const uint32_t*>(p->tree_mask);
  a.status = reinterpret_cast<int32_t*>(ws);
  a.sb_check = a.status + 1;                         // header words 1 .. waves_per_group
  a.sb_words = pl.waves_per_group;
  a.ws_ml = reinterpret_cast<float*>(ws + 256);
  a.ws_o = reinterpret_cast<float*>(ws + 256 + ml_bytes);
  a.num_seqs = p->num_seqs;
  a.num_tokens = p->num_tokens;
  a.Hq = p->num_q_heads;
  a.Hkv = p->num_kv_heads;
  a.G = p->num_q_heads / p->num_kv_heads;
  a.num_blocks = p->num_blocks;
  a.mbps = p->max_blocks_per_seq;
  a.window = p->sliding_window;
  a.max_ctx = max_ctx;
  a.max_q = (int32_t)query_bound(p);
  a.S = pl.num_segments;
  a.steps_per_seg = pl.steps_per_segment;
  a.n_steps = pl.num_steps;
  a.worklist = pl.worklist;
  a.target_items = pl.target_items;
  a.max_sps = pav::max_steps_per_segment(p->block_size);
  a.scale_log2 = scale * 1.4426950408889634f;
  a.page_layout = p->page_layout;
  a.direct = pl.direct;
  a.out = out;
  a.small_groups = pl.small_groups;

  hipStream_t st = static_cast<hipStream_t>(p->stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(p->prof_event_begin);
  hipEvent_t e1 = static_cast<hipEvent_t>(p->prof_event_end);
  const dim3 grid(pl.grid[0], pl.grid[1], pl.grid[2]);
  const int rb = pl.row_blocks;
  hipError_t e;
  if (u8_entry)
    e = pav::launch_segment_u8(a, p->q_dtype, p->head_dim, p->block_size, rb, grid, st, e0, e1);
  else if (p->kv_dtype == PA_F16)
    e = pav::launch_segment_f16(a, p->head_dim, p->block_size, rb, grid, st, e0, e1);
  else
    e = pav::launch_segment_bf16(a, p->head_dim, p->block_size, rb, grid, st, e0, e1);
  if (e == hipErrorNotSupported) return PA_ERR_UNSUPPORTED;
  if (e != hipSuccess) return PA_ERR_HIP;
  pav::CombineArgs c;
  c.seg = a;
  c.out = out;
  c.num_tokens = p->num_tokens;
  c.Hq = p->num_q_heads;
  // The segment grid's x dimension is the KV head and workgroups reach the X
  // XCDs round-robin by linear id, so the workgroups of KV head h ran on the
  // XCDs congruent to h modulo gcd(X, Hkv) (all on XCD h mod X when X
  // divides Hkv): put the pair's combine workgroup on one of those.
  int g = device_xccs();
  for (int b = p->num_kv_heads; b != 0;) {
    const int t = g % b;
    g = b;
    b = t;
  }
  c.xcds = g > 1 ? g : 0;
  c.head_dim = p->head_dim;
  if (pl.direct)
    e = pav::launch_finish(c, p->q_dtype, pl.combine_threads, dim3(pl.combine_grid[0]), st);
  else
    e = pav::launch_combine(c, p->q_dtype, p->head_dim, pl.combine_threads, dim3(pl.combine_grid[0]), st);
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

int run_append(const void* k_new, const void* v_new, void* k, void* v, void* ksz, void* vsz,
               const int32_t* bt, const int32_t* past_lens, const int32_t* sb,
               const pa_verify_params* p, bool u8_entry) {
  if (!p) return PA_ERR_INVALID_ARG;
  // the positions written must have a block-table entry: plan for the whole row
  const int64_t max_pos = (int64_t)p->max_blocks_per_seq * p->block_size;
  int rc = validate(p, (int32_t)std::min<int64_t>(max_pos, INT32_MAX), u8_entry);
  if (rc) return rc;
  if (!k_new || !v_new || !k || !v || !bt || !past_lens || !sb) return PA_ERR_INVALID_ARG;
  if (u8_entry && (!ksz || !vsz)) return PA_ERR_INVALID_ARG;
  const uintptr_t ce = u8_entry ? 1 : 2;                      // bytes per cache element
  if (!aligned(k_new, 2) || !aligned(v_new, 2) || !aligned(k, ce) || !aligned(v, ce) ||
      !aligned(ksz, 2) || !aligned(vsz, 2) || !aligned(bt, 4) || !aligned(past_lens, 4) ||
      !aligned(sb, 4))
    return PA_ERR_INVALID_ARG;
  if (!p->workspace || !aligned(p->workspace, 4) || p->workspace_bytes < sizeof(int32_t))
    return PA_ERR_WORKSPACE;
  if (p->num_tokens > 2147483647 / 2) return PA_ERR_UNSUPPORTED;
  pav::AppendArgs a;
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k;
  a.v_cache = v;
  a.ksz = ksz;
  a.vsz = vsz;
  a.bt = bt;
  a.past_lens = past_lens;
  a.sb = sb;
  a.status = static_cast<int32_t*>(p->workspace);
  a.num_seqs = p->num_seqs;
  a.num_tokens = p->num_tokens;
  a.Hkv = p->num_kv_heads;
  a.bs = p->block_size;
  a.mbps = p->max_blocks_per_seq;
  a.num_blocks = p->num_blocks;
  a.max_q = (int32_t)query_bound(p);
  a.page_layout = p->page_layout;
  const hipError_t e = pav::launch_append(a, p->q_dtype, p->kv_dtype, p->head_dim,
                                          static_cast<hipStream_t>(p->stream));
  return e == hipSuccess ? PA_OK : PA_ERR_HIP;
}

}  // namespace

extern "C" {

int pa_verify_make_plan(const pa_verify_params* p, int32_t max_context_len, int32_t num_cus,
                        pa_verify_plan* plan) {
  if (!plan || num_cus < 1) return PA_ERR_INVALID_ARG;
  const bool u8 = p && p->kv_dtype == PA_U8;
  int rc = validate(p, max_context_len, u8);
  if (rc) return rc;
  return make_plan(p, max_context_len, num_cus, plan);
}

size_t pa_verify_workspace_bytes(const pa_verify_params* p, int32_t max_context_len) {
  const bool u8 = p && p->kv_dtype == PA_U8;
  if (validate(p, max_context_len, u8)) return 0;
  int cus = 0;
  if (device_cus(&cus)) return 0;
  pa_verify_plan pl;
  if (make_plan(p, max_context_len, cus, &pl)) return 0;
  return pl.workspace_bytes;
}

int pa_verify_forward(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* past_lens,
                      const int32_t* subsequence_begins, int32_t max_context_len, float scale,
                      void* out, const pa_verify_params* p) {
  return run(q, k_cache, v_cache, nullptr, nullptr, block_tables, past_lens, subsequence_begins,
             max_context_len, scale, out, p, false);
}

int pa_verify_forward_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* past_lens,
                              const int32_t* subsequence_begins, int32_t max_context_len,
                              float scale, void* out, const pa_verify_params* p) {
  return run(q, k_cache, v_cache, nullptr, nullptr, block_tables, past_lens, subsequence_begins,
             max_context_len, scale, out, p, false, scratch_address);
}

int pa_verify_forward_u8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                         const void* k_scale_zp, const void* v_scale_zp,
                         const int32_t* block_tables, const int32_t* past_lens,
                         const int32_t* subsequence_begins, int32_t max_context_len, float scale,
                         void* out, const pa_verify_params* p) {
  return run(q, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables, past_lens,
             subsequence_begins, max_context_len, scale, out, p, true);
}

int pa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* block_tables, const int32_t* past_lens,
                 const int32_t* subsequence_begins, const pa_verify_params* p) {
  return run_append(k_new, v_new, k_cache, v_cache, nullptr, nullptr, block_tables, past_lens,
                    subsequence_begins, p, false);
}

int pa_kv_append_u8(const void* k_new, const void* v_new, uint8_t* k_cache, uint8_t* v_cache,
                    void* k_scale_zp, void* v_scale_zp, const int32_t* block_tables,
                    const int32_t* past_lens, const int32_t* subsequence_begins,
                    const pa_verify_params* p) {
  return run_append(k_new, v_new, k_cache, v_cache, k_scale_zp, v_scale_zp, block_tables,
                    past_lens, subsequence_begins, p, true);
}

int pa_verify_read_status(const pa_verify_params* p, int32_t* device_status) {
  if (!p || !device_status || !p->workspace || p->workspace_bytes < sizeof(int32_t))
    return PA_ERR_INVALID_ARG;
  hipStream_t st = static_cast<hipStream_t>(p->stream);
  if (hipStreamSynchronize(st) != hipSuccess) return PA_ERR_HIP;
  int32_t w = 0;
  if (hipMemcpy(&w, p->workspace, sizeof w, hipMemcpyDeviceToHost) != hipSuccess) return PA_ERR_HIP;
  if (w != 0 && hipMemset(p->workspace, 0, sizeof w) != hipSuccess) return PA_ERR_HIP;
  *device_status = w == 0 ? PA_OK : PA_ERR_DEVICE_CONTRACT;
  return PA_OK;
}

const char* pa_verify_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_INVALID_ARG: return "PA_ERR_INVALID_ARG: null or misaligned pointer, or inconsistent sizes";
    case PA_ERR_UNSUPPORTED: return "PA_ERR_UNSUPPORTED: head_dim, block_size, group size or dtype combination not built";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing, misaligned or smaller than pa_verify_workspace_bytes";
    case PA_ERR_HIP: return "PA_ERR_HIP: HIP runtime call or kernel launch failed";
    case PA_ERR_DEVICE_CONTRACT: return "PA_ERR_DEVICE_CONTRACT: device metadata violated the contract";
  }
  return "unknown pa_status";
}

}  // extern "C"
