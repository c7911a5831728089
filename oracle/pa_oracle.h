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
  const void* k_cache;                /* [nb][Hkv][bs * D], tiled pages (see pa_oracle.c) */
  const void* v_cache;                /* [nb][Hkv][bs * D], tiled pages */
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
} pa_oracle_args;

/* out: fp64 [num_tokens][Hq][D], or [num_pairs][D] when pairs is given.
 * Returns PA_ORACLE_OK, or an error code without touching out. */
int pa_oracle_forward(const pa_oracle_args* a, double* out);
int pa_oracle_num_threads(void);

#endif
