/*
 * Plain CPU oracle of the Lightning Indexer backward pass fused with its KL loss.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: it exists so that tests/, the smoke check and the bench's
 * CPU baseline can compare the HIP library against the definition.  It shares
 * no header, helper, table or constant with the HIP library.
 *
 * Definition followed (npu_sparse_lightning_indexer_grad_kl_loss page, 计算公式
 * items 1-4, and its parameter list), for every query token t with the valid
 * entries j of sparse_indices[t] (keys s_j; the -1 padding is skipped):
 *   1. index scores   I_j = sum_h w[t,h] * ReLU(S_h,j),  S_h,j = qi[t,h,:] . ki[s_j,:]
 *   2. main attention P_g,j = exp(scale * (q[t,g,:] . k[s_j,:] + qr[t,g,:] . kr[s_j,:])
 *                              - softmax_max[t,g]) / softmax_sum[t,g]
 *      (the softmax of item 2 recomputed from the statistics the attention
 *      forward saved; scale_value in place of 1/sqrt(d));
 *      target p_j = sum_g P_g,j / sum_j' sum_g P_g,j'  (head sum, then L1
 *      normalisation along the context);
 *   3. loss_t = D_KL(p || Softmax(I)) = sum_j p_j (log p_j - log pi_j), pi = Softmax(I)
 *      over the selected keys, 0 log 0 = 0; the loss is the sum over t;
 *   4. dI_j = pi_j - p_j;  dW[t,h] = sum_j dI_j ReLU(S_h,j);
 *      dS_h,j = dI_j w[t,h] [S_h,j > 0];  dqi[t,h,:] = sum_j dS_h,j ki[s_j,:];
 *      dki[s,:] += sum_{t,h,j: s_j = s} dS_h,j qi[t,h,:].
 * Everything in fp64 with one fixed summation order.
 */
#ifndef LI_GRAD_ORACLE_H
#define LI_GRAD_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* layouts (query and key sides alike) */
#define LIOG_BSND 0
#define LIOG_TND 1
/* element types */
#define LIOG_BF16 0
#define LIOG_FP32 2
#define LIOG_FP16 3
#define LIOG_FP64 4

typedef struct {
  int32_t batch;          /* B */
  int32_t s1, s2;         /* BSND query / key lengths */
  int32_t layout;         /* LIOG_BSND | LIOG_TND */
  int32_t n_main;         /* G: main-attention query heads (one key head) */
  int32_t d_main;         /* main-attention head dim */
  int32_t d_rope;         /* rope dim (0: no rope inputs) */
  int32_t n_idx;          /* index query heads */
  int32_t d_idx;          /* index head dim */
  int32_t topk;           /* entries per sparse_indices row */
  int32_t dtype;          /* element type of q, k, q_rope, k_rope, qi, ki */
  int32_t w_dtype;        /* element type of w */
  double scale;           /* scale_value */
} liog_problem;

typedef struct {
  const void* q;          /* [B,S1,G,Dm] or [T1,G,Dm] */
  const void* k;          /* [B,S2,1,Dm] or [T2,1,Dm] */
  const void* q_rope;     /* [.., G, Dr] or NULL when d_rope == 0 */
  const void* k_rope;     /* [.., 1, Dr] or NULL */
  const void* qi;         /* [B,S1,Ni,Di] or [T1,Ni,Di] */
  const void* ki;         /* [B,S2,1,Di] or [T2,1,Di] */
  const void* w;          /* [B,S1,Ni] or [T1,Ni] */
  const int32_t* sparse_indices;   /* [rows, topk]: sequence-local key positions, -1 = none */
  const float* softmax_max;        /* [rows, G] */
  const float* softmax_sum;        /* [rows, G] */
  const int32_t* cu_seqlens_q;     /* TND: B inclusive prefix sums */
  const int32_t* cu_seqlens_k;
} liog_inputs;

/* Query rows (B*S1 or T1) and key rows (B*S2 or T2). */
int64_t liog_num_rows(const liog_problem* p, const liog_inputs* in);
int64_t liog_num_keys(const liog_problem* p, const liog_inputs* in);

/* The loss of every row (loss_rows [rows]) and the gradients: d_qi [rows, Ni, Di],
 * d_ki [keys, Di], d_w [rows, Ni], all fp64 and fully overwritten.  Any output
 * pointer may be NULL to skip it.  Rows are shared by `nthreads` POSIX threads;
 * d_ki is accumulated afterwards, each key's sum over the rows in row order (the
 * threads split the keys), so no bit depends on the thread count.  Returns 0, or
 * -1 on an invalid argument. */
int liog_backward(const liog_problem* p, const liog_inputs* in, double* loss_rows,
                  double* d_qi, double* d_ki, double* d_w, int nthreads);

/* The same outputs for the listed rows only (no d_ki): loss [nrows], d_qi [nrows, Ni, Di],
 * d_w [nrows, Ni].  One thread.  Returns 0, or -1 on an invalid argument. */
int liog_backward_rows(const liog_problem* p, const liog_inputs* in, const int64_t* rows,
                       int64_t nrows, double* loss, double* d_qi, double* d_w);

/* Exact value of one element code (pins). */
double liog_decode(int dtype, const void* ptr, int64_t index);

#ifdef __cplusplus
}
#endif
#endif
