/*
 * Plain CPU oracle of the Lightning Indexer forward pass.
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's CPU
 * baseline to check the HIP library against.  Never linked into the product.
 *
 * Each step follows the pages directly, with no tiling, blocking, radix or
 * histogram tricks:
 *   1. lengths per batch: BSND dims, TND from inclusive cu_seqlens (lightning_indexer
 *      page, Constraints: cumulative valid tokens of this and the preceding batches),
 *      PA from seqused_k (same page: seqused_k must be passed with the paged layout);
 *   2. visible keys: mask_mode 0 = all keys of the batch; mask_mode 3 =
 *      rightDownCausal, the lower triangle anchored at the bottom-right corner
 *      (npu_lightning_indexer_pto page, sparse_mode), read as
 *      s <= i + S2_b - S1_b, diagonal included (a token sees itself and the
 *      tokens before it: lightning_indexer page, Function step 2).
 *      Compressed keys (cmp_ratio r > 1, lightning_indexer page, parameters and
 *      Example): key j stands for the r original positions j*r .. j*r + r - 1,
 *      the batch has S2_b*r + cmp_residual_k[b] original keys (the residual ones
 *      trail, not yet compressed), local row i is original position
 *      i + S2_b*r + res_b - S1_b, and it sees key j when the whole block lies at
 *      or before that position (a reading: the pages give the shapes only);
 *   3. score I = sum_h w[h] * max(0, sum_d q[h,d] * k[s,d]) in fp64 (the formula of
 *      the npu_lightning_indexer_pto page; steps 1-3 of the lightning_indexer page);
 *      fp8 codes are multiplied by their per-token descale;
 *   4. rank visible keys by (I descending, s ascending), keep n = min(topk, |V|),
 *      pad the rest with -1 / -inf (lightning_indexer page, Constraints); with
 *      output_idx_offset each kept index of batch b is written plus offset[b]
 *      (aclnnLightningIndexerV2 page, 约束说明: a positive index offset).
 */
#include "li_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- element decoding (exact) ------------------------------------------ */

static double dec_bf16(uint16_t u) {
  uint32_t bits = ((uint32_t)u) << 16;   /* bf16 is the top half of an fp32 */
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double dec_fp16(uint16_t u) {
  int sign = (u >> 15) & 1;
  int e = (u >> 10) & 31;
  int m = u & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);                 /* subnormal */
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

/* OCP e4m3fn: 1 sign, 4 exponent (bias 7), 3 mantissa bits; no infinities,
 * S.1111.111 is NaN, largest finite 448. */
static double dec_e4m3(uint8_t c) {
  int sign = (c >> 7) & 1;
  int e = (c >> 3) & 15;
  int m = c & 7;
  double v;
  if (e == 0) v = ldexp((double)m, -9);                  /* subnormal: m * 2^-9 */
  else if (e == 15 && m == 7) v = NAN;
  else v = ldexp((double)(8 + m), e - 10);               /* (1 + m/8) * 2^(e-7) */
  return sign ? -v : v;
}

double lio_decode(int dtype, const void* ptr, int64_t index) {
  switch (dtype) {
    case LIO_BF16: return dec_bf16(((const uint16_t*)ptr)[index]);
    case LIO_FP16: return dec_fp16(((const uint16_t*)ptr)[index]);
    case LIO_E4M3: return dec_e4m3(((const uint8_t*)ptr)[index]);
    case LIO_FP32: return (double)((const float*)ptr)[index];
    default: return NAN;
  }
}

/* ---- lengths and addressing -------------------------------------------- */

static int64_t prev_cu(const int32_t* cu, int b) { return b == 0 ? 0 : cu[b - 1]; }

static int seqlen_q(const lio_problem* p, const lio_inputs* in, int b) {
  if (p->layout_q == LIO_TND) return (int)(in->cu_seqlens_q[b] - prev_cu(in->cu_seqlens_q, b));
  return p->s1;
}

static int seqlen_k(const lio_problem* p, const lio_inputs* in, int b) {
  if (p->layout_k == LIO_TND) return (int)(in->cu_seqlens_k[b] - prev_cu(in->cu_seqlens_k, b));
  if (p->layout_k == LIO_PA_BSND) return in->seqused_k[b];
  return p->s2;
}

/* global query token index of local row i of batch b */
static int64_t q_token(const lio_problem* p, const lio_inputs* in, int b, int i) {
  if (p->layout_q == LIO_TND) return prev_cu(in->cu_seqlens_q, b) + i;
  return (int64_t)b * p->s1 + i;
}

/* element offset of key s of batch b, and the index of its descale */
static int64_t k_offset(const lio_problem* p, const lio_inputs* in, int b, int s, int64_t* dsc) {
  if (p->layout_k == LIO_PA_BSND) {
    int blk = in->block_table[(int64_t)b * p->max_blocks_per_seq + s / p->block_size];
    int row = s % p->block_size;
    *dsc = (int64_t)blk * p->block_size + row;
    return (int64_t)blk * p->k_block_stride + (int64_t)row * p->d;
  }
  int64_t tok = (p->layout_k == LIO_TND) ? prev_cu(in->cu_seqlens_k, b) + s
                                         : (int64_t)b * p->s2 + s;
  *dsc = tok;
  return tok * p->d;
}

int64_t lio_num_rows(const lio_problem* p, const lio_inputs* in) {
  if (p->batch <= 0) return 0;
  if (p->layout_q == LIO_TND) return in->cu_seqlens_q[p->batch - 1];
  return (int64_t)p->batch * p->s1;
}

int lio_row_coords(const lio_problem* p, const lio_inputs* in, int64_t row, int* b, int* i) {
  if (row < 0 || row >= lio_num_rows(p, in)) return -1;
  if (p->layout_q == LIO_TND) {
    for (int bb = 0; bb < p->batch; ++bb) {
      if (row < in->cu_seqlens_q[bb]) {
        *b = bb;
        *i = (int)(row - prev_cu(in->cu_seqlens_q, bb));
        return 0;
      }
    }
    return -1;
  }
  *b = (int)(row / p->s1);
  *i = (int)(row % p->s1);
  return 0;
}

int lio_visible_count(const lio_problem* p, const lio_inputs* in, int b, int i) {
  int S1 = seqlen_q(p, in, b), S2 = seqlen_k(p, in, b);
  if (p->mask_mode == 0) return S2;
  if (p->cmp_ratio > 1) {
    /* count the compressed keys whose whole block of original positions ends
     * at or before the row's original position */
    long long r = p->cmp_ratio;
    long long pos = (long long)i + (long long)S2 * r + in->cmp_residual_k[b] - S1;
    int n = 0;
    for (int j = 0; j < S2; ++j)
      if ((long long)j * r + r - 1 <= pos) ++n;
    return n;
  }
  long long last = (long long)i + S2 - S1;     /* largest visible key */
  if (last < 0) return 0;
  if (last >= S2) return S2;
  return (int)(last + 1);
}

/* ---- scores -------------------------------------------------------------- */

/* fp64 score of key s for a row whose decoded q (n1 x d) and w (n1) are given.
 * krow: scratch of d doubles that receives the decoded (descaled) key row, which
 * every head then reads. */
static double score_row_key(const lio_problem* p, const lio_inputs* in, const double* qrow,
                            const double* wrow, int b, int s, double* krow) {
  int64_t dsc;
  int64_t koff = k_offset(p, in, b, s, &dsc);
  double kd = (p->qk_dtype == LIO_E4M3) ? (double)in->k_descale[dsc] : 1.0;
  for (int e = 0; e < p->d; ++e) krow[e] = lio_decode(p->qk_dtype, in->k, koff + e) * kd;
  double total = 0.0;
  for (int h = 0; h < p->n1; ++h) {
    double x = 0.0;
    for (int d = 0; d < p->d; ++d) {
      x += qrow[(int64_t)h * p->d + d] * krow[d];
    }
    double r = x > 0.0 ? x : 0.0;                      /* ReLU */
    total += wrow[h] * r;
  }
  return total;
}

static void load_row(const lio_problem* p, const lio_inputs* in, int b, int i, double* qrow,
                     double* wrow) {
  int64_t t = q_token(p, in, b, i);
  double qd = (p->qk_dtype == LIO_E4M3) ? (double)in->q_descale[t] : 1.0;
  for (int64_t e = 0; e < (int64_t)p->n1 * p->d; ++e)
    qrow[e] = lio_decode(p->qk_dtype, in->q, t * p->n1 * p->d + e) * qd;
  for (int h = 0; h < p->n1; ++h) wrow[h] = lio_decode(p->w_dtype, in->w, t * p->n1 + h);
}

double lio_score(const lio_problem* p, const lio_inputs* in, int b, int i, int s) {
  double* qrow = (double*)malloc(sizeof(double) * (size_t)p->n1 * p->d);
  double* wrow = (double*)malloc(sizeof(double) * (size_t)p->n1);
  double* krow = (double*)malloc(sizeof(double) * (size_t)p->d);
  load_row(p, in, b, i, qrow, wrow);
  double v = score_row_key(p, in, qrow, wrow, b, s, krow);
  free(qrow);
  free(wrow);
  free(krow);
  return v;
}

/* ---- ranking ------------------------------------------------------------- */

typedef struct {
  double score;
  int32_t key;
} cand;

static int cand_cmp(const void* a, const void* b) {
  const cand* x = (const cand*)a;
  const cand* y = (const cand*)b;
  if (x->score > y->score) return -1;      /* higher score first */
  if (x->score < y->score) return 1;
  return (x->key > y->key) - (x->key < y->key);   /* then smaller key first */
}

static void one_row(const lio_problem* p, const lio_inputs* in, int64_t row, int32_t* oi,
                    float* ov, double* qrow, double* wrow, double* krow) {
  int b = 0, i = 0;
  int nvis = 0;
  if (lio_row_coords(p, in, row, &b, &i) == 0) nvis = lio_visible_count(p, in, b, i);
  cand* c = NULL;
  if (nvis > 0) {
    c = (cand*)malloc(sizeof(cand) * (size_t)nvis);
    load_row(p, in, b, i, qrow, wrow);
    /* the visible keys are exactly 0 .. nvis-1 under both mask modes */
    for (int s = 0; s < nvis; ++s) {
      c[s].score = score_row_key(p, in, qrow, wrow, b, s, krow);
      c[s].key = s;
    }
    qsort(c, (size_t)nvis, sizeof(cand), cand_cmp);
  }
  int n = nvis < p->topk ? nvis : p->topk;
  int32_t off = in->output_idx_offset && nvis > 0 ? in->output_idx_offset[b] : 0;
  for (int j = 0; j < p->topk; ++j) {
    if (j < n) {
      oi[j] = c[j].key + off;
      ov[j] = (float)c[j].score + 0.0f;              /* one RNE rounding; -0 -> +0 */
    } else {
      oi[j] = -1;
      ov[j] = -INFINITY;
    }
  }
  free(c);
}

typedef struct {
  const lio_problem* p;
  const lio_inputs* in;
  const int64_t* rows;
  int64_t nrows;
  int32_t* out_idx;
  float* out_val;
  int tid, nthreads;
} job;

static void* worker(void* arg) {
  job* jb = (job*)arg;
  const lio_problem* p = jb->p;
  double* qrow = (double*)malloc(sizeof(double) * (size_t)p->n1 * p->d);
  double* wrow = (double*)malloc(sizeof(double) * (size_t)p->n1);
  double* krow = (double*)malloc(sizeof(double) * (size_t)p->d);
  for (int64_t j = jb->tid; j < jb->nrows; j += jb->nthreads) {
    int64_t row = jb->rows ? jb->rows[j] : j;
    one_row(p, jb->in, row, jb->out_idx + j * p->topk, jb->out_val + j * p->topk, qrow, wrow,
            krow);
  }
  free(qrow);
  free(wrow);
  free(krow);
  return NULL;
}

int lio_forward(const lio_problem* p, const lio_inputs* in, const int64_t* rows, int64_t nrows,
                int32_t* out_idx, float* out_val, int nthreads) {
  if (!p || !in || !out_idx || !out_val) return -1;
  if (p->n1 <= 0 || p->d <= 0 || p->topk <= 0 || p->batch < 0) return -1;
  if (p->mask_mode != 0 && p->mask_mode != 3) return -1;
  if (p->layout_q == LIO_TND && !in->cu_seqlens_q) return -1;
  if (p->layout_k == LIO_TND && !in->cu_seqlens_k) return -1;
  if (p->layout_k == LIO_PA_BSND && (!in->seqused_k || !in->block_table || p->block_size <= 0))
    return -1;
  if (p->qk_dtype == LIO_E4M3 && (!in->q_descale || !in->k_descale)) return -1;
  if (p->cmp_ratio > 1 && p->mask_mode == 3 && !in->cmp_residual_k) return -1;
  if (!rows) nrows = lio_num_rows(p, in);
  if (nthreads <= 0) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  job jobs[256];
  if (nthreads == 1) {
    jobs[0] = (job){p, in, rows, nrows, out_idx, out_val, 0, 1};
    worker(&jobs[0]);
    return 0;
  }
  int started = 0, rc = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (job){p, in, rows, nrows, out_idx, out_val, t, nthreads};
    if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) {
      rc = -1;
      break;
    }
    ++started;
  }
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  return rc;
}
