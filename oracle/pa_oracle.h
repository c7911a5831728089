/*
 * pa_oracle.h — interface of the fp64 CPU oracle (test infrastructure only;
 * the library never includes or links it).
 */
#ifndef PA_ORACLE_H
#define PA_ORACLE_H

#include <stdint.h>

enum { PA_ORACLE_F16 = 0, PA_ORACLE_BF16 = 1, PA_ORACLE_U8 = 2, PA_ORACLE_F64 = 3 };
enum { PA_ORACLE_OK = 0, PA_ORACLE_ERR_ARG = 1, PA_ORACLE_ERR_META = 2 };

typedef struct pa_oracle_args {
  int32_t num_seqs, num_tokens, num_q_heads, num_kv_heads, head_dim, block_size;
  int32_t num_blocks, max_blocks_per_seq, sliding_window, max_context_len;
  int32_t q_dtype, kv_dtype;          /* element codes above */
  double scale;
  const void* q;                      /* [num_tokens][Hq][D] */
  const void* k_cache;                /* [nb][Hkv][bs * D] pages (see pa_oracle.c) */
  const void* v_cache;                /* [nb][Hkv][bs * D] pages */
  const void* k_scale_zp;             /* f16 [nb][Hkv][bs][2], u8 only */
  const void* v_scale_zp;
  const int32_t* block_tables;        /* [num_seqs][max_blocks_per_seq] */
  const int32_t* past_lens;           /* [num_seqs] */
  const int32_t* subsequence_begins;  /* [num_seqs + 1] */
  const uint32_t* tree_mask;          /* optional [num_tokens]: bit j of token b0 + i lets row
                                         i see new token j of its sequence (bit i implied);
                                         NULL = causal rows; needs sliding_window == 0 */
  const int32_t* pairs;               /* optional [num_pairs][2] (token, q head) subset */
  int64_t num_pairs;
  int32_t num_threads;                /* 0 = all online host cores */
  int32_t page_layout;                /* 0: tiled pages (see pa_oracle.c); 1: every page
                                         row-major [slot][d] for K and V */
} pa_oracle_args;

/* Writing the new tokens into the cache (the step before the attention):
 * token b_s + i of sequence s goes to position L_s + i.  k_new / v_new are
 * [num_tokens][Hkv][D] in new_dtype (f16 or bf16 codes).  For an f16/bf16
 * cache (kv_dtype == new_dtype) the values are stored as they are; for a u8
 * cache each (token, KV head) vector is quantised (pa_oracle.c,
 * quantize_row) and its f16 (scale, zero point) stored beside it.  Caches
 * are updated in place; only the written slots change. */
typedef struct pa_oracle_append_args {
  int32_t num_seqs, num_tokens, num_kv_heads, head_dim, block_size;
  int32_t num_blocks, max_blocks_per_seq;
  int32_t new_dtype, kv_dtype;
  const void* k_new;
  const void* v_new;
  void* k_cache;                      /* [nb][Hkv][bs * D] pages */
  void* v_cache;
  uint16_t* k_scale_zp;               /* f16 [nb][Hkv][bs][2], u8 only */
  uint16_t* v_scale_zp;
  const int32_t* block_tables;
  const int32_t* past_lens;
  const int32_t* subsequence_begins;
  int32_t page_layout;                /* as in pa_oracle_args */
} pa_oracle_append_args;

int pa_oracle_kv_append(const pa_oracle_append_args* a);

/* One row's u8 quantisation (exposed for the tests): codes[D], f16 bits of
 * scale and zero point. */
void pa_oracle_quantize_row(const float* x, int D, uint8_t* codes, uint16_t* scale_bits,
                            uint16_t* zp_bits);

/* out: fp64 [num_tokens][Hq][D], or [num_pairs][D] when pairs is given.
 * Returns PA_ORACLE_OK, or an error code without touching out. */
int pa_oracle_forward(const pa_oracle_args* a, double* out);
int pa_oracle_num_threads(void);

#endif
