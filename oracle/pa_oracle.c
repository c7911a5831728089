/*
 * pa_oracle.c — the CPU oracle for paged verify attention.  TEST
 * INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
 * baseline use it; the library never does.  It shares no code, header,
 * table or helper with the GPU path.
 *
 * It is the plain definition of the operation, in fp64, written as loops:
 *
 *  - New query token i (0-based inside its sequence) of a sequence with
 *    past_len L attends to cache positions below L + i + 1: OpenVINO issue
 *    #38153 "[GPU] PagedAttention with 2-4 query tokens per sequence
 *    (speculative decoding verify) is ~8x slower than single-token decode",
 *    section "Performance issue description" (the suggested key limit).
 *  - The op metadata (past_lens, subsequence_begins, max_context_len, one
 *    block table per sequence) and the u8 KV cache: same issue, section
 *    "Step-by-step reproduction".
 *  - A sliding-window layer (window 1024 in the model measured) keeps only the
 *    last W positions, the token itself included: SGLang discussion #36314
 *    "FROZEN_KV_MTP slower than no-spec on Gemma 4 (SWA hybrid)", section
 *    "Observation 3".  Reading: W counts the token itself.
 *  - Grouped-query attention: q head h reads KV head h / (Hq / Hkv).  The
 *    pages only name "GQA read-once"; consecutive grouping is the reading.
 *  - Tree verify (optional): the new tokens of a sequence form a tree of
 *    drafts and row i sees the cached past plus the new tokens its mask
 *    names — its ancestors — instead of all earlier ones: OpenVINO #38153
 *    "Performance issue description" (the neighbouring tree-mask verify case)
 *    and "The 140x Performance Gap" (a tree of draft tokens verified in one
 *    pass).  Reading: bit j of row i's mask admits new token j; bit i (the
 *    token itself) is always admitted; no sliding window with a tree.
 *  - Softmax is taken over scale * q.k, two passes (max, then exp-sum), no
 *    segmentation, no online rescaling: the segmented GPU reduction must
 *    reach the same value up to rounding order (vLLM article "speculative
 *    decoding net loss", passage on the 18 fixed-input kernel cases).
 *
 * Layouts (the library's C ABI defines them; restated here on purpose):
 *   q [num_tokens][Hq][D]; k and v [nb][Hkv][page], each page holding the
 *   block_size x D elements of one (block, KV head) in the order of
 *   k_offset / v_offset below (row-major for layout 1; for layout 0 tiled
 *   when block_size % 16 == 0, K row-major and V d-major for pages of 1, 2,
 *   4 or 8 slots); scale/zero point
 *   [nb][Hkv][bs][2] (f16); block_tables [num_seqs][mbps].  Requires
 *   D % 32 == 0 (D % 64 == 0 for u8).
 * Element codes: 0 = f16 bits, 1 = bf16 bits, 2 = u8 code with f16
 * (scale, zero point), 3 = fp64 value (test-only input form).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

#include "pa_oracle.h"

/* IEEE binary16 bit pattern -> exact double. */
static double dec_f16(uint16_t b) {
  int sign = (b >> 15) & 1;
  int exp = (b >> 10) & 0x1f;
  int man = b & 0x3ff;
  double v;
  if (exp == 0) {
    v = ldexp((double)man, -24);                   /* subnormal: man * 2^-24 */
  } else if (exp == 31) {
    v = man ? NAN : INFINITY;
  } else {
    v = ldexp((double)(man | 0x400), exp - 25);    /* (1024 + man) * 2^(exp-15-10) */
  }
  return sign ? -v : v;
}

/* bfloat16 bit pattern -> exact double (bf16 is the top half of a float32). */
static double dec_bf16(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

static double dec_elem(const void* base, size_t idx, int code) {
  switch (code) {
    case PA_ORACLE_F16: return dec_f16(((const uint16_t*)base)[idx]);
    case PA_ORACLE_BF16: return dec_bf16(((const uint16_t*)base)[idx]);
    case PA_ORACLE_F64: return ((const double*)base)[idx];
    default: return NAN;
  }
}

/* Offsets of element (slot, d) inside one page.  Row-major pages (layout 1):
 * [slot][d] for K and V.  Tiled pages (layout 0): pages of 1-8 slots hold K
 * as [slot][d] and V as [d][slot]; larger ones are sub-tiles of 16 slots, in
 * each of which K is ordered [d/32][(d%32)/8][slot%16][d%8] (u8: [d/64][(d%64)/16]
 * [slot%16][d%16]) and V [d/32][(slot%16)/4][d%16][(d%32)/16][slot%4] (u8:
 * [d/64][(slot%16)/4][d%16][(d%64)/16][slot%4]). */
static size_t k_offset(int slot, int d, int D, int u8, int bs, int layout) {
  if (layout == 1) return (size_t)slot * D + d;    /* row-major page */
  if (bs < 16) return (size_t)slot * D + d;        /* small pages: [slot][d] */
  const size_t st = (size_t)(slot / 16), m = (size_t)(slot % 16);
  if (u8) return (((st * (D / 64) + d / 64) * 4 + (d % 64) / 16) * 16 + m) * 16 + d % 16;
  return (((st * (D / 32) + d / 32) * 4 + (d % 32) / 8) * 16 + m) * 8 + d % 8;
}

static size_t v_offset(int slot, int d, int D, int u8, int bs, int layout) {
  if (layout == 1) return (size_t)slot * D + d;    /* row-major page */
  if (bs < 16) return (size_t)d * bs + slot;       /* small pages: [d][slot] */
  const size_t st = (size_t)(slot / 16), qq = (size_t)((slot % 16) / 4);
  if (u8) return ((((st * (D / 64) + d / 64) * 4 + qq) * 16 + d % 16) * 4 + (d % 64) / 16) * 4 + slot % 4;
  return ((((st * (D / 32) + d / 32) * 4 + qq) * 16 + d % 16) * 2 + (d % 32) / 16) * 4 + slot % 4;
}

/* One KV value.  For u8, code u of (block, head, slot) means (u - zp) * scale
 * with the per-token per-KV-head f16 pair stored next to the cache. */
static double kv_value(const pa_oracle_args* a, const void* cache, const void* sz,
                       size_t elem_idx, size_t slot_idx) {
  if (a->kv_dtype == PA_ORACLE_U8) {
    const uint16_t* p = (const uint16_t*)sz;
    double s = dec_f16(p[2 * slot_idx + 0]);
    double zp = dec_f16(p[2 * slot_idx + 1]);
    return ((double)((const uint8_t*)cache)[elem_idx] - zp) * s;
  }
  return dec_elem(cache, elem_idx, a->kv_dtype);
}

/* Check the metadata the way the definition needs it: returns 0 when every
 * sequence has 1 <= T, 0 <= L, L + T <= max_context_len, a well-formed
 * subsequence_begins and in-range block ids for every position it reads. */
static int check_args(const pa_oracle_args* a) {
  if (a->num_seqs < 1 || a->num_q_heads < 1 || a->num_kv_heads < 1 || a->head_dim < 1 ||
      a->block_size < 1 || a->num_q_heads % a->num_kv_heads != 0)
    return PA_ORACLE_ERR_ARG;
  if ((a->block_size % 16 != 0 && a->block_size != 1 && a->block_size != 2 && a->block_size != 4 &&
       a->block_size != 8) ||
      a->head_dim % (a->kv_dtype == PA_ORACLE_U8 ? 64 : 32) != 0)
    return PA_ORACLE_ERR_ARG;                       /* the page layouts need these */
  if (!a->q || !a->k_cache || !a->v_cache || !a->block_tables || !a->past_lens ||
      !a->subsequence_begins)
    return PA_ORACLE_ERR_ARG;
  if (a->kv_dtype == PA_ORACLE_U8 && (!a->k_scale_zp || !a->v_scale_zp)) return PA_ORACLE_ERR_ARG;
  if (a->tree_mask && a->sliding_window > 0) return PA_ORACLE_ERR_ARG;
  if (a->page_layout != 0 && a->page_layout != 1) return PA_ORACLE_ERR_ARG;
  if (a->subsequence_begins[0] != 0 || a->subsequence_begins[a->num_seqs] != a->num_tokens)
    return PA_ORACLE_ERR_META;
  for (int s = 0; s < a->num_seqs; ++s) {
    int T = a->subsequence_begins[s + 1] - a->subsequence_begins[s];
    int L = a->past_lens[s];
    if (T < 1 || L < 0 || (int64_t)L + T > a->max_context_len) return PA_ORACLE_ERR_META;
    int nblk = (L + T + a->block_size - 1) / a->block_size;
    if (nblk > a->max_blocks_per_seq) return PA_ORACLE_ERR_META;
    int lo_first = a->sliding_window > 0 ? L + 1 - a->sliding_window : 0;
    if (lo_first < 0) lo_first = 0;
    for (int b = lo_first / a->block_size; b < nblk; ++b) {
      int id = a->block_tables[(size_t)s * a->max_blocks_per_seq + b];
      if (id < 0 || id >= a->num_blocks) return PA_ORACLE_ERR_META;
    }
  }
  return PA_ORACLE_OK;
}

/* Does query token i (of a sequence with past_len L and T new tokens) see
 * cache position t?  Causal rows: t in [lo, L + i + 1).  Tree rows: every
 * past position, and new token j = t - L when bit j of the row's mask is set
 * or j == i. */
static int visible(const pa_oracle_args* a, int n, int i, int L, int T, int lo, int t) {
  if (t < lo) return 0;
  if (!a->tree_mask) return t < L + i + 1;
  if (t < L) return 1;
  const int j = t - L;
  if (j >= T) return 0;
  return j == i || ((a->tree_mask[n] >> j) & 1u);
}

/* out[row][:] for query token n, q head h: the definition, two-pass softmax. */
static void attend_one(const pa_oracle_args* a, int n, int h, double* z, double* out_row) {
  const int D = a->head_dim, bs = a->block_size, Hq = a->num_q_heads, Hkv = a->num_kv_heads;
  int s = 0;
  while (!(a->subsequence_begins[s] <= n && n < a->subsequence_begins[s + 1])) ++s;
  const int i = n - a->subsequence_begins[s];      /* index of the token inside its sequence */
  const int T = a->subsequence_begins[s + 1] - a->subsequence_begins[s];
  const int L = a->past_lens[s];
  const int hi = a->tree_mask ? L + T : L + i + 1;  /* candidate keys [lo, hi) */
  int lo = 0;
  if (a->sliding_window > 0) {
    lo = L + i + 1 - a->sliding_window;
    if (lo < 0) lo = 0;
  }
  const int g = h / (Hq / Hkv);                     /* KV head serving q head h */
  const int32_t* table = a->block_tables + (size_t)s * a->max_blocks_per_seq;
  const size_t q_off = ((size_t)n * Hq + h) * D;

  const int u8 = a->kv_dtype == PA_ORACLE_U8;

  /* pass 1: logits and their max */
  double m = -INFINITY;
  for (int t = lo; t < hi; ++t) {
    if (!visible(a, n, i, L, T, lo, t)) continue;
    const size_t blk = (size_t)table[t / bs];
    const int slot = t % bs;
    const size_t row = (blk * Hkv + g) * bs + slot; /* index of (blk, g, slot) */
    const size_t page = (blk * Hkv + g) * (size_t)bs * D;
    double dot = 0.0;
    for (int d = 0; d < D; ++d)
      dot += dec_elem(a->q, q_off + d, a->q_dtype) *
             kv_value(a, a->k_cache, a->k_scale_zp, page + k_offset(slot, d, D, u8, bs, a->page_layout), row);
    z[t - lo] = a->scale * dot;
    if (z[t - lo] > m) m = z[t - lo];
  }
  /* pass 2: weights, their sum, and the weighted sum of V rows */
  double Z = 0.0;
  for (int d = 0; d < D; ++d) out_row[d] = 0.0;
  for (int t = lo; t < hi; ++t) {
    if (!visible(a, n, i, L, T, lo, t)) continue;
    const double w = exp(z[t - lo] - m);
    Z += w;
    const size_t blk = (size_t)table[t / bs];
    const int slot = t % bs;
    const size_t row = (blk * Hkv + g) * bs + slot;
    const size_t page = (blk * Hkv + g) * (size_t)bs * D;
    for (int d = 0; d < D; ++d) {
      const size_t vidx = page + v_offset(slot, d, D, u8, bs, a->page_layout);
      out_row[d] += w * kv_value(a, a->v_cache, a->v_scale_zp, vidx, row);
    }
  }
  for (int d = 0; d < D; ++d) out_row[d] /= Z;
}

typedef struct {
  const pa_oracle_args* a;
  double* out;
  int64_t num_items;
  int tid, nthreads;
} worker_t;

static void* worker(void* arg) {
  worker_t* w = (worker_t*)arg;
  const pa_oracle_args* a = w->a;
  double* z = (double*)malloc(sizeof(double) * (size_t)(a->max_context_len > 0 ? a->max_context_len : 1));
  if (!z) return (void*)1;
  for (int64_t it = w->tid; it < w->num_items; it += w->nthreads) {
    int n, h;
    if (a->pairs) {
      n = a->pairs[2 * it];
      h = a->pairs[2 * it + 1];
    } else {
      n = (int)(it / a->num_q_heads);
      h = (int)(it % a->num_q_heads);
    }
    attend_one(a, n, h, z, w->out + (size_t)it * a->head_dim);
  }
  free(z);
  return NULL;
}

int pa_oracle_num_threads(void) {
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

int pa_oracle_forward(const pa_oracle_args* a, double* out) {
  if (!a || !out) return PA_ORACLE_ERR_ARG;
  int rc = check_args(a);
  if (rc) return rc;
  int64_t items = a->pairs ? a->num_pairs : (int64_t)a->num_tokens * a->num_q_heads;
  if (a->pairs) {
    for (int64_t it = 0; it < items; ++it)
      if (a->pairs[2 * it] < 0 || a->pairs[2 * it] >= a->num_tokens || a->pairs[2 * it + 1] < 0 ||
          a->pairs[2 * it + 1] >= a->num_q_heads)
        return PA_ORACLE_ERR_ARG;
  }
  int nt = a->num_threads > 0 ? a->num_threads : pa_oracle_num_threads();
  if (nt > items) nt = items > 0 ? (int)items : 1;
  pthread_t th[256];
  worker_t ws[256];
  if (nt > 256) nt = 256;
  for (int t = 0; t < nt; ++t) {
    ws[t] = (worker_t){a, out, items, t, nt};
    if (pthread_create(&th[t], NULL, worker, &ws[t]) != 0) return PA_ORACLE_ERR_ARG;
  }
  int bad = 0;
  for (int t = 0; t < nt; ++t) {
    void* r = NULL;
    pthread_join(th[t], &r);
    if (r) bad = 1;
  }
  return bad ? PA_ORACLE_ERR_ARG : PA_ORACLE_OK;
}

/* ---------------------------------------------------------------------------
 * Appending the new tokens, with u8 quantisation for a u8 cache.
 *
 * The cache holds u8 KV with f16 compute (OpenVINO #38153, "Step-by-step
 * reproduction"), quantised per token per KV head, asymmetric, with an f16
 * scale and an f16 zero point.  The pages fix no formula; the reading taken:
 * over the row's D values in fp32,
 *     scale = (max - min) / 255,  rounded to f16 -> s
 *     zero point = -min / s,      rounded to f16 -> z
 *     code = clamp(round_half_even(x / s + z), 0, 255)
 * every step an IEEE fp32 operation; a constant row (max == min), or one
 * whose scale rounds to 0 in f16, takes s = 1 and z = f16(-min).
 * ------------------------------------------------------------------------- */

/* float32 -> IEEE binary16 bits, round to nearest even (finite inputs; values
 * beyond the f16 range become infinity). */
static uint16_t f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const uint32_t a = u & 0x7fffffffu;
  if (a >= 0x7f800000u) return (uint16_t)(sign | 0x7c00u | (a > 0x7f800000u ? 0x200u : 0u));
  const double v = (double)fabsf(f);              /* exact */
  if (v >= 65520.0) return (uint16_t)(sign | 0x7c00u);   /* rounds past the largest finite */
  /* scale so that one unit is the f16 spacing at v, round half to even */
  int e;
  frexp(v, &e);                                   /* v = m * 2^e, m in [0.5, 1) */
  int q = e - 11;                                 /* spacing 2^(e-11) for normals */
  if (q < -24) q = -24;                           /* subnormal spacing */
  const double t = ldexp(v, -q);
  double r = floor(t);
  const double frac = t - r;
  if (frac > 0.5 || (frac == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  const double rv = ldexp(r, q);                  /* rounded value, exact */
  if (rv == 0.0) return sign;
  int e2;
  frexp(rv, &e2);
  if (e2 - 1 < -14) return (uint16_t)(sign | (uint16_t)ldexp(rv, 24));   /* subnormal */
  const int exp16 = e2 - 1 + 15;
  const uint32_t man = (uint32_t)(ldexp(rv, 11 - e2) - 1024.0);
  return (uint16_t)(sign | (uint16_t)(exp16 << 10) | (uint16_t)man);
}

static float f16_to_f32(uint16_t b) { return (float)dec_f16(b); }

void pa_oracle_quantize_row(const float* x, int D, uint8_t* codes, uint16_t* scale_bits,
                            uint16_t* zp_bits) {
  float mn = x[0], mx = x[0];
  for (int d = 1; d < D; ++d) {
    if (x[d] < mn) mn = x[d];
    if (x[d] > mx) mx = x[d];
  }
  uint16_t sb = 0x3c00u;                          /* 1.0 */
  uint16_t zb;
  const float range = mx - mn;
  const uint16_t s_try = f32_to_f16(range / 255.0f);
  if (mx != mn && s_try != 0) {
    sb = s_try;
    zb = f32_to_f16(-mn / f16_to_f32(sb));
  } else {
    zb = f32_to_f16(-mn);
  }
  const float s = f16_to_f32(sb), z = f16_to_f32(zb);
  for (int d = 0; d < D; ++d) {
    const float y = x[d] / s + z;
    float r = rintf(y);                           /* default mode: nearest, ties to even */
    if (r < 0.0f) r = 0.0f;
    if (r > 255.0f) r = 255.0f;
    codes[d] = (uint8_t)r;
  }
  *scale_bits = sb;
  *zp_bits = zb;
}

int pa_oracle_kv_append(const pa_oracle_append_args* a) {
  if (!a || !a->k_new || !a->v_new || !a->k_cache || !a->v_cache || !a->block_tables ||
      !a->past_lens || !a->subsequence_begins)
    return PA_ORACLE_ERR_ARG;
  const int u8 = a->kv_dtype == PA_ORACLE_U8;
  if (a->new_dtype != PA_ORACLE_F16 && a->new_dtype != PA_ORACLE_BF16) return PA_ORACLE_ERR_ARG;
  if (!u8 && a->kv_dtype != a->new_dtype) return PA_ORACLE_ERR_ARG;
  if (a->page_layout != 0 && a->page_layout != 1) return PA_ORACLE_ERR_ARG;
  if (u8 && (!a->k_scale_zp || !a->v_scale_zp)) return PA_ORACLE_ERR_ARG;
  const int D = a->head_dim, bs = a->block_size, Hkv = a->num_kv_heads;
  if ((bs % 16 != 0 && bs != 1 && bs != 2 && bs != 4 && bs != 8) || D % (u8 ? 64 : 32) != 0)
    return PA_ORACLE_ERR_ARG;
  if (a->subsequence_begins[0] != 0 || a->subsequence_begins[a->num_seqs] != a->num_tokens)
    return PA_ORACLE_ERR_META;
  float* row = (float*)malloc(sizeof(float) * (size_t)D);
  uint8_t* codes = (uint8_t*)malloc((size_t)D);
  if (!row || !codes) {
    free(row);
    free(codes);
    return PA_ORACLE_ERR_ARG;
  }
  int rc = PA_ORACLE_OK;
  for (int s = 0; s < a->num_seqs && rc == PA_ORACLE_OK; ++s) {
    const int b0 = a->subsequence_begins[s], T = a->subsequence_begins[s + 1] - b0;
    const int L = a->past_lens[s];
    if (T < 0 || L < 0) {
      rc = PA_ORACLE_ERR_META;
      break;
    }
    for (int i = 0; i < T; ++i) {
      const int pos = L + i;
      if (pos / bs >= a->max_blocks_per_seq) {
        rc = PA_ORACLE_ERR_META;
        break;
      }
      const int blk = a->block_tables[(size_t)s * a->max_blocks_per_seq + pos / bs];
      if (blk < 0 || blk >= a->num_blocks) {
        rc = PA_ORACLE_ERR_META;
        break;
      }
      const int slot = pos % bs;
      for (int g = 0; g < Hkv; ++g) {
        const size_t src = ((size_t)(b0 + i) * Hkv + g) * D;
        const size_t page = ((size_t)blk * Hkv + g) * (size_t)bs * D;
        const size_t srow = ((size_t)blk * Hkv + g) * bs + slot;
        for (int kv = 0; kv < 2; ++kv) {
          const uint16_t* in = (const uint16_t*)(kv ? a->v_new : a->k_new);
          void* cache = kv ? a->v_cache : a->k_cache;
          if (!u8) {
            for (int d = 0; d < D; ++d) {
              const size_t off = page + (kv ? v_offset(slot, d, D, 0, bs, a->page_layout)
                                                : k_offset(slot, d, D, 0, bs, a->page_layout));
              ((uint16_t*)cache)[off] = in[src + d];
            }
            continue;
          }
          for (int d = 0; d < D; ++d) row[d] = (float)dec_elem(in, src + d, a->new_dtype);
          uint16_t sb, zb;
          pa_oracle_quantize_row(row, D, codes, &sb, &zb);
          for (int d = 0; d < D; ++d) {
            const size_t off = page + (kv ? v_offset(slot, d, D, 1, bs, a->page_layout)
                                                : k_offset(slot, d, D, 1, bs, a->page_layout));
            ((uint8_t*)cache)[off] = codes[d];
          }
          uint16_t* sz = kv ? a->v_scale_zp : a->k_scale_zp;
          sz[2 * srow + 0] = sb;
          sz[2 * srow + 1] = zb;
        }
      }
    }
  }
  free(row);
  free(codes);
  return rc;
}

