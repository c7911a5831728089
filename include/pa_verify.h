/*
 * pa_verify.h — C ABI of libpa_verify.so: paged attention for the verify step
 * of speculative decoding on MI355X (gfx950).
 *
 * What the operation computes.  A batch holds num_seqs sequences.  Sequence s
 * brings T_s = subsequence_begins[s+1] - subsequence_begins[s] new query
 * tokens (1 <= T_s <= 16) on top of past_len L_s = past_lens[s] cached tokens.
 * The paged KV cache already holds all L_s + T_s tokens of the sequence.  New
 * token i (0-based within its sequence) attends to cache positions
 * [lo_i, L_s + i + 1), with lo_i = 0 for a full-causal layer and
 * lo_i = max(0, L_s + i + 1 - W) for a sliding-window layer of window W
 * (the window counts the token itself).  Per query head h the result is
 *
 *     out[n, h, :] = sum_t softmax_t(scale * <q[n, h, :], k_t>) * v_t
 *
 * over those positions, where KV head floor(h / (Hq / Hkv)) serves q head h.
 * Tree verify (params->tree_mask) replaces the causal rule among the new
 * tokens: row i sees every past position and the new tokens its mask word
 * names (its ancestors in the draft tree) plus itself.
 *
 * Sources (cited by page title and section):
 *  - The per-token key limit past_len + i + 1, the op metadata (past_lens,
 *    subsequence_begins, max_context_len, one block table per sequence) and a
 *    u8 KV cache with f16 compute: OpenVINO issue #38153 "[GPU] PagedAttention
 *    with 2-4 query tokens per sequence (speculative decoding verify) is ~8x
 *    slower than single-token decode", sections "Performance issue
 *    description" and "Step-by-step reproduction".
 *  - The KV scan split into segments reduced in parallel, and segment buffers
 *    that must be sized per query token, not per sequence: the vLLM article
 *    "speculative decoding net loss" (dual-radeon-vllm), passages on the
 *    use_3d gate, the segment-buffer geometry and vllm#45450.
 *  - The sliding window of 1024 and page size 64 of the SWA-hybrid model:
 *    SGLang discussion #36314 "FROZEN_KV_MTP slower than no-spec on Gemma 4
 *    (SWA hybrid)", sections "Environment" and "Observation 3".
 *  - Tree-mask verify with up to 9-16 draft tokens as the neighbouring case:
 *    OpenVINO issue #38153, "Performance issue description" (#34644), and
 *    "The 140x Performance Gap" (magik.net), section "The Real Discovery"
 *    (a draft tree of 9 queries verified in one pass).
 *  - Graph replay must stay intact (no allocation, no host sync in a call):
 *    the same vLLM article, torch-profiler trace passage (hipGraphLaunch).
 *
 * Memory layouts (contiguous, caller-owned device memory):
 *  q, out        [num_tokens, Hq, D]  row-major, f16 or bf16 (out dtype == q dtype)
 *  k_cache,      [num_blocks, Hkv, page]: one page of block_size x D elements
 *  v_cache       per (block, KV head).  A page is block_size/16 sub-tiles of 16
 *                slots; inside a sub-tile the elements are stored in the order
 *                the gfx950 MFMA operands consume them, so that each wavefront
 *                load reads 1 KB of contiguous memory.  Element (slot s, dim d)
 *                of a page sits at element offset
 *     K f16/bf16: ((((s/16)*(D/32) + d/32)*4 + (d%32)/8)*16 + s%16)*8 + d%8
 *     V f16/bf16: (((((s/16)*(D/32) + d/32)*4 + (s%16)/4)*16 + d%16)*2 + (d%32)/16)*4 + s%4
 *     K u8:       ((((s/16)*(D/64) + d/64)*4 + (d%64)/16)*16 + s%16)*16 + d%16
 *     V u8:       (((((s/16)*(D/64) + d/64)*4 + (s%16)/4)*16 + d%16)*4 + (d%64)/16)*4 + s%4
 *                Pages of 1, 2, 4 or 8 slots hold K row-major (s*D + d) and V
 *                d-major (d*block_size + s), for every cache dtype.
 *                With params->page_layout = PA_PAGES_ROW_MAJOR every page is
 *                instead row-major for K and V, element (s, d) at s*D + d: the
 *                conventional [num_blocks, Hkv, block_size, D] cache.  The
 *                tiled order is the default because every load instruction then
 *                reads 1 KB of contiguous memory straight into MFMA operand
 *                order, while row-major V has to be reordered through LDS.
 *                Measured on MI355X, us per call tiled vs row-major: 32k
 *                context, 32 q / 8 KV heads, head_dim 128, f16: 26.2 vs 27.8;
 *                bf16 head_dim 256 (16 KV heads): 84.8 vs 102.9; ragged bf16
 *                batch: 64.1 vs 69.3; u8 head_dim 256: 20.7 vs 26.7.
 *  k_scale_zp,   [num_blocks, Hkv, block_size, 2]     f16 (scale, zero_point) per
 *  v_scale_zp    token per KV head, u8 variant only; dequant = (u - zp) * scale
 *  block_tables  [num_seqs, max_blocks_per_seq] int32 physical block ids
 *  past_lens     [num_seqs] int32
 *  subsequence_begins [num_seqs + 1] int32, cumulative, [0] == 0,
 *                [num_seqs] == num_tokens
 *
 * Alignment (the kernels use 16-byte vector accesses).  Forward calls: q,
 * out, k_cache, v_cache, k_scale_zp, v_scale_zp and the workspace 16-byte
 * aligned; block_tables, past_lens, subsequence_begins and tree_mask 4
 * bytes.  Append calls: the new K/V rows, the caches and the
 * scale/zero-point arrays 2 bytes (the u8 caches 1), the int32 arrays and the
 * workspace 4 bytes.  A misaligned pointer is PA_ERR_INVALID_ARG (a
 * misaligned workspace PA_ERR_WORKSPACE), returned before anything is
 * enqueued.  hipMalloc and torch's allocator give 256-byte aligned storage;
 * a view that starts inside a storage may not be.
 *
 * Ownership and behaviour.  The library never allocates, frees or retains a
 * pointer past the call and never synchronises (except pa_verify_read_status).
 * A forward call enqueues exactly two kernels (segment kernel, then combine
 * kernel; with one segment, the segment kernel writes the output and a
 * check kernel takes the combine's place) on params->stream, so it can be
 * captured in a HIP graph.  Calls are
 * stateless and thread-safe; calls that share one workspace must be ordered
 * on one stream.  No C++ exception crosses this ABI.
 *
 * Errors.  Host-checkable problems return a nonzero pa_status before anything
 * is enqueued and leave `out` untouched.  Problems that only the device can see
 * (T_s outside [1, max_query_len], L_s < 0, L_s + T_s > max_context_len, a physical block id
 * outside [0, num_blocks), non-monotone subsequence_begins, and with an f16 q
 * a u8 V scale whose weighted product overflows f16, see pa_verify_forward_u8)
 * set the sticky device status word PA_ERR_DEVICE_CONTRACT in the workspace
 * and make the affected sequence's output rows NaN; pa_verify_read_status
 * reports it.
 */
#ifndef PA_VERIFY_H
#define PA_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,      /* null or misaligned pointer, non-positive size, inconsistent sizes */
  PA_ERR_UNSUPPORTED = 2,      /* valid but not built: D, block_size, group size, dtype combo */
  PA_ERR_WORKSPACE = 3,        /* workspace missing, misaligned or smaller than pa_verify_workspace_bytes */
  PA_ERR_HIP = 4,              /* a HIP runtime call or kernel launch failed */
  PA_ERR_DEVICE_CONTRACT = 5   /* device-side metadata violated the contract (see above) */
} pa_status;

typedef enum pa_page_layout {
  PA_PAGES_TILED = 0,      /* the MFMA-operand order above (default) */
  PA_PAGES_ROW_MAJOR = 1   /* every page [block_size][D] for K and V */
} pa_page_layout;

typedef enum pa_dtype {
  PA_F16 = 0,
  PA_BF16 = 1,
  PA_U8 = 2   /* KV only: asymmetric per-token per-KV-head u8 with f16 scale and zero point */
} pa_dtype;

/* Sizes and options of one call.  Supported: head_dim in {64, 128, 256},
 * block_size in {1, 2, 4, 8, 16, 32, 64}, group size G = Hq/Hkv in
 * {1, 2, 4, 8}, dtype pairs (q, kv) = (f16, f16), (bf16, bf16), (f16, u8),
 * (bf16, u8), and up to 16 new tokens per sequence with G * max_query_len
 * stacked rows of at most 64 for head_dim 64, 48 for 128, 32 for u8 at 256
 * and 16 for f16/bf16 at 256 (16 for every head_dim when block_size < 16);
 * T_s <= max_query_len is checked per sequence on the device. */
typedef struct pa_verify_params {
  int32_t num_seqs;            /* sequences in the batch, 1 ..= 65535 */
  int32_t num_tokens;          /* == subsequence_begins[num_seqs], >= num_seqs */
  int32_t num_q_heads;         /* Hq */
  int32_t num_kv_heads;        /* Hkv, divides Hq */
  int32_t head_dim;            /* D */
  int32_t block_size;          /* tokens per page */
  int32_t num_blocks;          /* physical pages in the pool (device bounds check) */
  int32_t max_blocks_per_seq;  /* row stride of block_tables; >= ceil(max_context_len / block_size) */
  int32_t sliding_window;      /* W; 0 = full causal */
  int32_t num_segments;        /* 0 = planner decides; > 0 forces the segment count (clamped) */
  int32_t q_dtype;             /* pa_dtype of q and out: PA_F16 or PA_BF16 */
  int32_t kv_dtype;            /* pa_dtype of the caches: q_dtype, or PA_U8 (u8 entry point) */
  int32_t max_query_len;       /* bound on T_s, 1..16; 0 = min(4, num_tokens - num_seqs + 1).
                                  Sizes the kernel's row blocks (G * bound rows, in blocks
                                  of 16), so pass the real bound (the draft length) */
  void* workspace;             /* device scratch >= pa_verify_workspace_bytes; its first 4 bytes
                                  are the sticky device status word: zero them once at allocation
                                  (the rest is rewritten by every call) */
  size_t workspace_bytes;
  void* stream;                /* hipStream_t to enqueue on; NULL = the null stream */
  void* prof_event_begin;      /* optional hipEvent_t stamped when the segment kernel starts */
  void* prof_event_end;        /* optional hipEvent_t stamped when the segment kernel ends; both
                                  are set by the kernel's own dispatch (hipExtLaunchKernel),
                                  so their elapsed time is the kernel's duration */
  const void* tree_mask;       /* optional device uint32 [num_tokens]: tree verify.  Bit j of
                                  the word of token b_s + i lets that row see new token j of
                                  sequence s (cache position L_s + j) instead of the causal
                                  rule; the row's own bit is implied, bits >= T_s are ignored,
                                  every past position stays visible.  NULL = causal rows.
                                  Requires sliding_window == 0 (else PA_ERR_UNSUPPORTED) */
  int32_t page_layout;         /* pa_page_layout of k_cache and v_cache (forward and append
                                  calls); anything else is PA_ERR_INVALID_ARG */
} pa_verify_params;

/* The launch plan, a pure function of host scalars: segment count S, keys per
 * segment, grids and workspace size.  Exposed so callers and tests can see
 * what a call will launch. */
typedef struct pa_verify_plan {
  int32_t num_segments;        /* S: KV segments per (sequence, KV head) */
  int32_t steps_per_segment;   /* steps of keys_per_step keys in the longest segment; segment j
                                  covers steps [j*N/S, (j+1)*N/S) of num_steps = N */
  int32_t num_steps;           /* N: steps covering span */
  int32_t row_blocks;          /* 16-row blocks of stacked query rows the kernel is built with */
  int32_t worklist;            /* 1 for a batch of 2 .. min(target_items, 256) sequences: the
                                  grid is (Hkv, 1, chunks) and each workgroup takes one chunk
                                  of a work list the device builds from the sequence lengths
                                  (chunk size chosen so the chunks fill one round of
                                  target_items workgroups per KV head); 0: fixed segments,
                                  also for larger batches (every sequence has its own) */
  int32_t target_items;        /* work-list chunks per KV head the chunk size aims at */
  int32_t keys_per_step;       /* keys one wavefront consumes per loop iteration */
  int32_t span;                /* bound on keys any one sequence's rows touch */
  int32_t waves_per_group;     /* wavefronts per segment workgroup */
  int32_t max_steps_per_segment; /* most steps one segment or work-list chunk may span: its
                                  block ids (one per page, plus one for a step that starts
                                  inside a page and one for the last page) fit the kernel's
                                  LDS table of 1040 ids (2080 for block_size 1) */
  int32_t grid[3];             /* segment kernel grid: (Hkv, num_seqs, S), z = S-1-j; work
                                  list: (Hkv, 1, chunks) */
  int32_t block_threads;       /* segment kernel workgroup size */
  int32_t combine_grid[3];     /* combine kernel grid (direct: the check kernel's) */
  int32_t combine_threads;     /* combine kernel workgroup size (direct: the check kernel's) */
  size_t workspace_bytes;      /* status word + per-token segment partials (direct: 256) */
  int32_t direct;              /* 1 when S == 1: the segment kernel normalises and writes the
                                  output rows itself (no partials), and a check kernel that
                                  turns every row NaN if subsequence_begins is broken runs
                                  in the combine kernel's place */
  int32_t small_groups;        /* for a direct call over short contexts (one row block, tiled
                                  pages of >= 16 slots): the segment workgroups' wavefronts,
                                  2 up to 16 steps, 4 up to 48 (more of them per CU); else 0 */
} pa_verify_plan;

/* Fill *plan for params p, host scalar max_context_len (>= max_s L_s + T_s)
 * and a compute-unit count num_cus (> 0).  No device access.  Returns PA_OK or
 * the same host-side error pa_verify_forward would return (except workspace). */
int pa_verify_make_plan(const pa_verify_params* p, int32_t max_context_len,
                        int32_t num_cus, pa_verify_plan* plan);

/* Workspace bytes a forward call with these params needs on the current
 * device (queries its compute-unit count once).  Returns 0 on invalid input
 * or when no device is present. */
size_t pa_verify_workspace_bytes(const pa_verify_params* p, int32_t max_context_len);

/* Paged verify attention, f16 or bf16 KV cache (kv_dtype == q_dtype).
 * q, k_cache, v_cache, out: device pointers in the layouts above.
 * block_tables, past_lens, subsequence_begins: device int32 arrays.
 * max_context_len: host scalar >= max over s of past_lens[s] + T_s; it sizes
 * the grid and workspace without reading device memory.
 * scale: multiplies q.k before the softmax (e.g. 1/sqrt(D)).
 * Returns PA_OK once both kernels are enqueued. */
int pa_verify_forward(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* past_lens,
                      const int32_t* subsequence_begins, int32_t max_context_len,
                      float scale, void* out, const pa_verify_params* p);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * pa_verify_forward with the same arguments, whose segment partials and
 * status word live in a static device array of the library instead of a
 * caller workspace (p->workspace and p->workspace_bytes are ignored).  The
 * array holds 32 MiB on each GPU the library runs on, until the process
 * ends; a call that needs more (pa_verify_workspace_bytes > 33554432)
 * returns PA_ERR_WORKSPACE before anything is enqueued.  The call allocates
 * nothing and enqueues the same two kernels.  All calls on one GPU share its
 * array: calls that may overlap on one GPU (other streams, other threads)
 * race and must be ordered by the caller.  The array's status word is never
 * reported: a device-side contract violation shows as NaN in the affected
 * rows of `out`.  The first call on each device resolves the array's address
 * (no allocation); make it outside graph capture. */
int pa_verify_forward_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* past_lens,
                              const int32_t* subsequence_begins, int32_t max_context_len,
                              float scale, void* out, const pa_verify_params* p);

/* The same operation over a u8 KV cache (kv_dtype == PA_U8): a cached value u
 * of token t, KV head g stands for (u - zp) * scale with (scale, zp) read as
 * f16 from k_scale_zp / v_scale_zp[block, g, slot, 0..1].  Dequantisation
 * follows that formula exactly in f32/f16 arithmetic inside the kernel.
 * Range: with an f16 q, the PV product takes each softmax weight (at most
 * 256 relative to the kernel's running reference) times the key's V scale as
 * an f16 operand, so V scales up to 255.875 (65504 / 256; a V row range up to
 * 65248 quantised by pa_kv_append_u8) always give the result.  A larger V
 * scale is outside the contract: where its product overflows f16, the rows
 * of that KV head become NaN and the device status word is set
 * (PA_ERR_DEVICE_CONTRACT); a wrong finite result is never returned.  A bf16
 * q has no such bound. */
int pa_verify_forward_u8(const void* q, const uint8_t* k_cache, const uint8_t* v_cache,
                         const void* k_scale_zp, const void* v_scale_zp,
                         const int32_t* block_tables, const int32_t* past_lens,
                         const int32_t* subsequence_begins, int32_t max_context_len,
                         float scale, void* out, const pa_verify_params* p);

/* Write the new tokens' K and V into their cache slots, the step before the
 * forward call reads them (OpenVINO issue #38153, "Step-by-step reproduction":
 * the op's cache holds the new tokens, u8 with f16 compute).  Token b_s + i
 * of sequence s goes to position L_s + i: block
 * block_tables[s][(L_s + i) / block_size], slot (L_s + i) % block_size, in
 * the page layout p->page_layout names.  k_new, v_new: device [num_tokens, Hkv, D] in
 * p->q_dtype.  Uses p's sizes, dtypes, max_query_len, stream and the status
 * word at the head of p->workspace (>= 4 bytes); not max_context_len.
 * Device-side contract violations (as for the forward call, with positions
 * bounded by max_blocks_per_seq * block_size) set the status word and write
 * nothing for that token.  subsequence_begins is checked as a whole by one
 * wavefront (a broken one sets the status word); each token is looked up as
 * the last s with subsequence_begins[s] <= token and written only if that
 * sequence's own checks pass, so a broken array can at most fill new-token
 * slots inside the block tables (the forward call then gives NaN rows).
 * Enqueues one kernel; enqueue it before the forward call on the same
 * stream. */
int pa_kv_append(const void* k_new, const void* v_new, void* k_cache, void* v_cache,
                 const int32_t* block_tables, const int32_t* past_lens,
                 const int32_t* subsequence_begins, const pa_verify_params* p);

/* The same into a u8 cache: each (token, KV head) vector x of D values is
 * quantised in IEEE fp32 steps, s = f16(range / 255), z = f16(-min / s),
 * code = clamp(round_half_even(x / s + z), 0, 255) (a constant row, or one
 * whose scale rounds to 0, takes s = 1, z = f16(-min)), and (s, z) is stored
 * in k_scale_zp / v_scale_zp.  Inputs must be finite and within the f16
 * range. */
int pa_kv_append_u8(const void* k_new, const void* v_new, uint8_t* k_cache, uint8_t* v_cache,
                    void* k_scale_zp, void* v_scale_zp, const int32_t* block_tables,
                    const int32_t* past_lens, const int32_t* subsequence_begins,
                    const pa_verify_params* p);

/* Synchronise p->stream, read the sticky device status word from
 * p->workspace into *device_status (PA_OK or PA_ERR_DEVICE_CONTRACT) and clear
 * it.  For tests and debugging; it blocks the host. */
int pa_verify_read_status(const pa_verify_params* p, int32_t* device_status);

/* Static, human-readable name of a pa_status value. */
const char* pa_verify_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* PA_VERIFY_H */
