/*
 * Plain CPU oracle of the Lightning Indexer backward pass fused with its KL
 * loss (npu_sparse_lightning_indexer_grad_kl_loss page, 计算公式 items 1-4).
 *
 * TEST INFRASTRUCTURE ONLY: used by tests/, the smoke check and the bench's CPU
 * baseline to check the HIP library against.  Never linked into the product.
 * The formulas and the readings taken where the page is silent are listed in
 * li_grad_oracle.h; each step below names the item it follows.
 */
#include "li_grad_oracle.h"

#include <math.h>
#include <pthread.h>
#include <stdlib.h>
#include <string.h>

/* ---- element decoding (exact) ------------------------------------------ */

static double dec_bf16(uint16_t u) {
  uint32_t bits = ((uint32_t)u) << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

static double dec_fp16(uint16_t u) {
  int sign = (u >> 15) & 1;
  int e = (u >> 10) & 31;
  int m = u & 1023;
  double v;
  if (e == 0) v = ldexp((double)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexp((double)(1024 + m), e - 25);
  return sign ? -v : v;
}

double liog_decode(int dtype, const void* ptr, int64_t index) {
  switch (dtype) {
    case LIOG_BF16: return dec_bf16(((const uint16_t*)ptr)[index]);
    case LIOG_FP16: return dec_fp16(((const uint16_t*)ptr)[index]);
    case LIOG_FP32: return (double)((const float*)ptr)[index];
    case LIOG_FP64: return ((const double*)ptr)[index];
    default: return NAN;
  }
}

/* ---- lengths ------------------------------------------------------------- */

static int64_t prev_cu(const int32_t* cu, int b) { return b == 0 ? 0 : cu[b - 1]; }

int64_t liog_num_rows(const liog_problem* p, const liog_inputs* in) {
  if (p->batch <= 0) return 0;
  if (p->layout == LIOG_TND) return in->cu_seqlens_q[p->batch - 1];
  return (int64_t)p->batch * p->s1;
}

int64_t liog_num_keys(const liog_problem* p, const liog_inputs* in) {
  if (p->batch <= 0) return 0;
  if (p->layout == LIOG_TND) return in->cu_seqlens_k[p->batch - 1];
  return (int64_t)p->batch * p->s2;
}

/* batch of query row `row`, and the token offset of that batch's keys */
static int row_batch(const liog_problem* p, const liog_inputs* in, int64_t row, int64_t* k_off,
                     int* s2) {
  int b;
  if (p->layout == LIOG_TND) {
    for (b = 0; b < p->batch; ++b)
      if (row < in->cu_seqlens_q[b]) break;
    *k_off = prev_cu(in->cu_seqlens_k, b);
    *s2 = (int)(in->cu_seqlens_k[b] - *k_off);
  } else {
    b = (int)(row / p->s1);
    *k_off = (int64_t)b * p->s2;
    *s2 = p->s2;
  }
  return b;
}

static double dot(int dt, const void* a, int64_t ia, const void* b, int64_t ib, int n) {
  double x = 0.0;
  for (int e = 0; e < n; ++e) x += liog_decode(dt, a, ia + e) * liog_decode(dt, b, ib + e);
  return x;
}

/* ---- one query row: items 1-4 except the d_ki accumulation ---------------- */

typedef struct {
  const liog_problem* p;
  const liog_inputs* in;
  double* loss_rows;
  double* d_qi;
  double* d_w;
  double* dI;        /* [rows, topk]: dI of each entry (0 for padding), for the d_ki pass */
  int tid, nthreads;
} job;

static void one_row(const liog_problem* p, const liog_inputs* in, int64_t t, double* loss_rows,
                    double* d_qi, double* d_w, double* dI_row) {
  const int K = p->topk, G = p->n_main, Ni = p->n_idx, Di = p->d_idx;
  int64_t k_off;
  int s2;
  row_batch(p, in, t, &k_off, &s2);
  const int32_t* sel = in->sparse_indices + t * K;
  double* I = (double*)calloc((size_t)K, sizeof(double));
  double* ph = (double*)calloc((size_t)K, sizeof(double));
  double* S = (double*)calloc((size_t)K * Ni, sizeof(double));
  int* valid = (int*)calloc((size_t)K, sizeof(int));
  int n = 0;
  for (int j = 0; j < K; ++j) {
    dI_row[j] = 0.0;
    valid[j] = sel[j] >= 0 && sel[j] < s2;
    n += valid[j];
  }
  if (d_w)
    for (int h = 0; h < Ni; ++h) d_w[t * Ni + h] = 0.0;
  if (d_qi)
    for (int64_t e = 0; e < (int64_t)Ni * Di; ++e) d_qi[t * Ni * Di + e] = 0.0;
  loss_rows[t] = 0.0;
  if (n == 0) goto done;

  for (int j = 0; j < K; ++j) {
    if (!valid[j]) continue;
    const int64_t key = k_off + sel[j];
    /* item 1: I_j = sum_h w_h ReLU(qi_h . ki_s) */
    double acc = 0.0;
    for (int h = 0; h < Ni; ++h) {
      double x = dot(p->dtype, in->qi, (t * Ni + h) * Di, in->ki, key * Di, Di);
      S[(int64_t)j * Ni + h] = x;
      acc += liog_decode(p->w_dtype, in->w, t * Ni + h) * (x > 0.0 ? x : 0.0);
    }
    I[j] = acc;
    /* item 2: the main attention's probabilities of this key, summed over heads */
    double psum = 0.0;
    for (int g = 0; g < G; ++g) {
      double x = dot(p->dtype, in->q, (t * G + g) * p->d_main, in->k, key * p->d_main, p->d_main);
      if (p->d_rope > 0)
        x += dot(p->dtype, in->q_rope, (t * G + g) * p->d_rope, in->k_rope, key * p->d_rope,
                 p->d_rope);
      psum += exp(p->scale * x - (double)in->softmax_max[t * G + g]) /
              (double)in->softmax_sum[t * G + g];
    }
    ph[j] = psum;
  }
  {
    /* item 2: L1 normalisation of the target along the selected keys */
    double z = 0.0;
    for (int j = 0; j < K; ++j)
      if (valid[j]) z += ph[j];
    /* item 3: pi = Softmax(I) over the selected keys; loss = KL(p || pi) */
    double mx = -INFINITY;
    for (int j = 0; j < K; ++j)
      if (valid[j] && I[j] > mx) mx = I[j];
    double se = 0.0;
    for (int j = 0; j < K; ++j)
      if (valid[j]) se += exp(I[j] - mx);
    const double lse = mx + log(se);
    double loss = 0.0;
    for (int j = 0; j < K; ++j) {
      if (!valid[j]) continue;
      const double pj = ph[j] / z;
      const double log_pi = I[j] - lse;
      if (pj > 0.0) loss += pj * (log(pj) - log_pi);
      /* item 4: dI = Softmax(I) - p */
      dI_row[j] = exp(log_pi) - pj;
    }
    loss_rows[t] = loss;
  }
  /* item 4: dW = dI @ ReLU(S)^T, dqi = dS @ ki with dS = dI w [S > 0] */
  for (int j = 0; j < K; ++j) {
    if (!valid[j]) continue;
    const int64_t key = k_off + sel[j];
    for (int h = 0; h < Ni; ++h) {
      const double x = S[(int64_t)j * Ni + h];
      if (d_w) d_w[t * Ni + h] += dI_row[j] * (x > 0.0 ? x : 0.0);
      if (d_qi && x > 0.0) {
        const double ds = dI_row[j] * liog_decode(p->w_dtype, in->w, t * Ni + h);
        for (int d = 0; d < Di; ++d)
          d_qi[(t * Ni + h) * Di + d] += ds * liog_decode(p->dtype, in->ki, key * Di + d);
      }
    }
  }
done:
  free(I);
  free(ph);
  free(S);
  free(valid);
}

static void* worker(void* arg) {
  job* jb = (job*)arg;
  const int64_t rows = liog_num_rows(jb->p, jb->in);
  for (int64_t t = jb->tid; t < rows; t += jb->nthreads)
    one_row(jb->p, jb->in, t, jb->loss_rows, jb->d_qi, jb->d_w, jb->dI + t * jb->p->topk);
  return NULL;
}

/* item 4: dki[s] += sum_h dS_h,j qi[t,h] over every (t, j) that selected s.  A
 * thread owns the key rows [k0, k1) and walks every row in order, so each key's
 * fp64 sum has one fixed order whatever the thread count. */
typedef struct {
  const liog_problem* p;
  const liog_inputs* in;
  const double* dI;
  double* d_ki;
  int64_t k0, k1;
} kjob;

static void* accumulate_dki(void* arg) {
  const kjob* kj = (const kjob*)arg;
  const liog_problem* p = kj->p;
  const liog_inputs* in = kj->in;
  const int K = p->topk, Ni = p->n_idx, Di = p->d_idx;
  const int64_t rows = liog_num_rows(p, in);
  for (int64_t e = kj->k0 * Di; e < kj->k1 * Di; ++e) kj->d_ki[e] = 0.0;
  for (int64_t t = 0; t < rows; ++t) {
    int64_t k_off;
    int s2;
    row_batch(p, in, t, &k_off, &s2);
    const int32_t* sel = in->sparse_indices + t * K;
    for (int j = 0; j < K; ++j) {
      if (sel[j] < 0 || sel[j] >= s2) continue;
      const int64_t key = k_off + sel[j];
      if (key < kj->k0 || key >= kj->k1) continue;
      for (int h = 0; h < Ni; ++h) {
        const double x = dot(p->dtype, in->qi, (t * Ni + h) * Di, in->ki, key * Di, Di);
        if (!(x > 0.0)) continue;
        const double ds = kj->dI[t * K + j] * liog_decode(p->w_dtype, in->w, t * Ni + h);
        for (int d = 0; d < Di; ++d)
          kj->d_ki[key * Di + d] += ds * liog_decode(p->dtype, in->qi, (t * Ni + h) * Di + d);
      }
    }
  }
  return NULL;
}

int liog_backward(const liog_problem* p, const liog_inputs* in, double* loss_rows,
                  double* d_qi, double* d_ki, double* d_w, int nthreads) {
  if (!p || !in || !in->qi || !in->ki || !in->w || !in->q || !in->k || !in->sparse_indices ||
      !in->softmax_max || !in->softmax_sum)
    return -1;
  if (p->batch < 0 || p->topk <= 0 || p->n_main <= 0 || p->n_idx <= 0 || p->d_idx <= 0 ||
      p->d_main <= 0 || p->d_rope < 0)
    return -1;
  if (p->d_rope > 0 && (!in->q_rope || !in->k_rope)) return -1;
  if (p->layout == LIOG_TND && (!in->cu_seqlens_q || !in->cu_seqlens_k)) return -1;
  const int64_t rows = liog_num_rows(p, in);
  double* lr = loss_rows ? loss_rows : (double*)malloc(sizeof(double) * (size_t)(rows ? rows : 1));
  double* dI = (double*)malloc(sizeof(double) * (size_t)(rows ? rows : 1) * p->topk);
  if (nthreads <= 0) nthreads = 1;
  if (nthreads > 256) nthreads = 256;
  pthread_t th[256];
  job jobs[256];
  int started = 0, rc = 0;
  for (int t = 0; t < nthreads; ++t) {
    jobs[t] = (job){p, in, lr, d_qi, d_w, dI, t, nthreads};
    if (nthreads == 1) {
      worker(&jobs[0]);
      break;
    }
    if (pthread_create(&th[t], NULL, worker, &jobs[t]) != 0) {
      rc = -1;
      break;
    }
    ++started;
  }
  for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  if (rc == 0 && d_ki) {
    const int64_t keys = liog_num_keys(p, in);
    kjob kjobs[256];
    started = 0;
    for (int t = 0; t < nthreads; ++t) {
      kjobs[t] = (kjob){p, in, dI, d_ki, keys * t / nthreads, keys * (t + 1) / nthreads};
      if (nthreads == 1) {
        accumulate_dki(&kjobs[0]);
        break;
      }
      if (pthread_create(&th[t], NULL, accumulate_dki, &kjobs[t]) != 0) {
        rc = -1;
        break;
      }
      ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(th[t], NULL);
  }
  free(dI);
  if (!loss_rows) free(lr);
  return rc;
}

int liog_backward_rows(const liog_problem* p, const liog_inputs* in, const int64_t* rows,
                       int64_t nrows, double* loss, double* d_qi, double* d_w) {
  if (!p || !in || !rows || !loss || !d_qi || !d_w) return -1;
  const int64_t total = liog_num_rows(p, in);
  const int K = p->topk, Ni = p->n_idx, Di = p->d_idx;
  double* l1 = (double*)malloc(sizeof(double) * (size_t)(total ? total : 1));
  double* q1 = (double*)malloc(sizeof(double) * (size_t)(total ? total : 1) * Ni * Di);
  double* w1 = (double*)malloc(sizeof(double) * (size_t)(total ? total : 1) * Ni);
  double* dI = (double*)malloc(sizeof(double) * (size_t)K);
  int rc = 0;
  for (int64_t r = 0; r < nrows; ++r) {
    const int64_t t = rows[r];
    if (t < 0 || t >= total) { rc = -1; break; }
    one_row(p, in, t, l1, q1, w1, dI);
    loss[r] = l1[t];
    memcpy(d_qi + r * Ni * Di, q1 + t * Ni * Di, sizeof(double) * (size_t)Ni * Di);
    memcpy(d_w + r * Ni, w1 + t * Ni, sizeof(double) * (size_t)Ni);
  }
  free(l1);
  free(q1);
  free(w1);
  free(dI);
  return rc;
}
