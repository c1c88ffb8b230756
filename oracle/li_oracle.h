/*
 * Plain CPU oracle of the Lightning Indexer forward pass (scores + top-k).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: it exists so that tests/, the smoke check and the bench's
 * CPU baseline can compare the HIP library against the definition.  It shares
 * no header, helper, table or constant with the HIP library.
 *
 * Definition followed (all pages agree on it):
 *   I[t,s] = sum_h w[t,h] * ReLU( q[t,h,:] . k[s,:] )
 *   - npu_lightning_indexer_pto page, formula under "功能说明" (per element),
 *   - lightning_indexer (CANN API) page, "Function", steps 1-3,
 *   - aclnnLightningIndexerV2 page, "计算公式" and "主要计算过程" steps 1-3,
 *   - npu_sparse_lightning_indexer_grad_kl_loss page, formula 1 ("Top-k value").
 * followed by a per-token top-k over the visible keys; invalid output slots
 * hold -1 (indices) and -inf (values) (lightning_indexer page, Constraints;
 * aclnnLightningIndexerV2 page, 约束说明).
 *
 * Scores are computed in fp64 with a fixed order (h ascending, d ascending),
 * ranked by (score descending, key index ascending), and the value written is
 * the fp64 score rounded once to fp32 (round to nearest even), with -0 turned
 * into +0.  Indices are sequence-local logical key positions (compressed-key
 * positions when cmp_ratio > 1), plus the batch's output index offset if given.
 */
#ifndef LI_ORACLE_H
#define LI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* layouts */
#define LIO_BSND 0
#define LIO_TND 1
#define LIO_PA_BSND 2
/* element types of q / k / w */
#define LIO_BF16 0
#define LIO_E4M3 1
#define LIO_FP32 2
#define LIO_FP16 3

typedef struct {
  int32_t batch;             /* B */
  int32_t s1, s2;            /* BSND query / key lengths (ignored by TND / PA sides) */
  int32_t n1;                /* query-index heads */
  int32_t d;                 /* head dim */
  int32_t topk;
  int32_t layout_q;          /* LIO_BSND | LIO_TND */
  int32_t layout_k;          /* LIO_BSND | LIO_TND | LIO_PA_BSND */
  int32_t mask_mode;         /* 0 = every key visible, 3 = right-down causal */
  int32_t qk_dtype;          /* LIO_BF16 | LIO_E4M3 | LIO_FP16 */
  int32_t w_dtype;           /* LIO_BF16 | LIO_FP32 */
  int32_t block_size;        /* PA only */
  int32_t max_blocks_per_seq;/* PA only: columns of block_table */
  int64_t k_block_stride;    /* PA only: elements between consecutive pool blocks */
  int32_t cmp_ratio;         /* original key positions per key (<= 1: no compression) */
} lio_problem;

typedef struct {
  const void* q;             /* [B,S1,N1,D] or [T1,N1,D], contiguous */
  const void* k;             /* [B,S2,1,D], [T2,1,D] contiguous; PA: pool, see k_block_stride */
  const void* w;             /* [B,S1,N1] or [T1,N1] */
  const float* q_descale;    /* e4m3 only: one per query token */
  const float* k_descale;    /* e4m3 only: one per key slot (PA: [num_blocks, block_size]) */
  const int32_t* cu_seqlens_q;  /* TND q: B inclusive prefix sums */
  const int32_t* cu_seqlens_k;  /* TND k: B inclusive prefix sums */
  const int32_t* seqused_k;     /* PA: keys per batch */
  const int32_t* block_table;   /* PA: [B, max_blocks_per_seq] */
  const int32_t* cmp_residual_k;     /* cmp_ratio > 1 with mask 3: [B], each in [0, cmp_ratio) */
  const int32_t* output_idx_offset;  /* NULL or [B]: added to every kept index of the batch */
} lio_inputs;

/* Number of query rows (B*S1 for BSND, T1 for TND). */
int64_t lio_num_rows(const lio_problem* p, const lio_inputs* in);

/* Computes the output rows listed in `rows` (global query-row ids: b*S1+i for
 * BSND, the packed token index for TND); rows == NULL means every row in order.
 * out_idx / out_val receive nrows x topk entries.  Uses `nthreads` POSIX
 * threads (<= 0: one).  Returns 0, or -1 on an invalid argument. */
int lio_forward(const lio_problem* p, const lio_inputs* in, const int64_t* rows, int64_t nrows,
                int32_t* out_idx, float* out_val, int nthreads);

/* fp64 score I of key s for local query row i of batch b (no masking). */
double lio_score(const lio_problem* p, const lio_inputs* in, int b, int i, int s);

/* |V(b,i)|: the number of keys visible to local row i of batch b. */
int lio_visible_count(const lio_problem* p, const lio_inputs* in, int b, int i);

/* Maps a global query-row id to (batch, local row); returns -1 if out of range. */
int lio_row_coords(const lio_problem* p, const lio_inputs* in, int64_t row, int* b, int* i);

/* Exact value of one element code, for the decoding pins. */
double lio_decode(int dtype, const void* ptr, int64_t index);

#ifdef __cplusplus
}
#endif
#endif
