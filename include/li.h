/*
 * li.h -- C ABI of the MI355X (gfx950) Lightning Indexer forward pass.
 *
 * What it computes.  For every query token t and every key s visible to it
 *
 *     I[t,s] = sum_h  w[t,h] * ReLU( q[t,h,:] . k[s,:] )          (D = 128)
 *
 * (npu_lightning_indexer_pto page, formula under "功能说明"; the lightning_indexer
 * CANN API page, "Function", steps 1-3; aclnnLightningIndexerV2 page, "计算公式"),
 * then, per token, the top-k visible keys: their positions go to sparse_indices and
 * their scores to sparse_values.  Slots past the number of visible keys hold -1 and
 * -inf (lightning_indexer page, Constraints).
 *
 * The work is split in two calls, like the pages' lightning_indexer_metadata +
 * lightning_indexer pair (lightning_indexer page, "Prototype": the metadata call
 * does the load balancing and must precede the indexer), and sizes are queried
 * first, like the two-phase aclnn interface (aclnnLightningIndexerV2 page: query
 * the workspace size, then execute).
 *
 * Conventions shared by every entry point:
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates no memory, never synchronises the host inside li_metadata or
 *    li_forward, and keeps no global mutable state: calls are thread-safe and
 *    may be captured in a HIP graph.  Work is enqueued on `stream` (0 = the null
 *    stream) and completes asynchronously.
 *  - Errors are reported only through li_status.  Every argument check that
 *    needs no device data runs before the first HIP call, so an invalid call
 *    enqueues nothing.  A problem with zero query rows returns LI_OK and
 *    launches nothing.
 *  - Data-dependent preconditions are not checked (undefined behaviour when
 *    violated): cu_seqlens non-decreasing with cu[B-1] equal to total_q /
 *    total_k; per-batch lengths <= max_seqlen_q / max_seqlen_k (the kernels
 *    hold each length to [0, max], so a longer one is cut short rather than
 *    read past the buffers sized from the maxima); seqused_k[b] <=
 *    max_blocks_per_seq * block_size; block_table entries in [0, num_blocks)
 *    for every block that holds a used key; descales finite and >= 0.
 *
 * Semantics fixed where the pages leave them open:
 *  - Indices are 0-based sequence-local LOGICAL key positions (not offsets into a
 *    packed TND tensor and not physical paged slots).
 *  - mask_mode 0: every key of the batch is visible.  mask_mode 3 (rightDownCausal,
 *    the lower triangle anchored at the bottom-right corner): local query row i of
 *    a batch with S1_b queries and S2_b keys sees keys s <= i + S2_b - S1_b.
 *  - Exactly n = min(topk, |visible|) valid entries, stored as the prefix
 *    [0, n) of each output row; among equal scores the smaller key index wins.
 *    The order inside the prefix is not specified (the pages' consumer gathers
 *    by index, which is order-free: aclnnSparseFlashAttentionGrad page,
 *    calculation formula), but it is deterministic: the same inputs give
 *    bitwise the same outputs.
 *  - No 1/sqrt(D) scale is applied.  fp8 inputs are e4m3fn codes whose real value is
 *    code * descale, with one fp32 descale per query token and per key slot.
 */
#ifndef LI_H
#define LI_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  LI_OK = 0,
  LI_ERR_INVALID_ARGUMENT = 1,   /* a value outside the documented range, a missing pointer */
  LI_ERR_UNSUPPORTED = 2,        /* valid for the pages but a shape whose working set does not
                                    fit the kernels (index or token counts past int32) */
  LI_ERR_WORKSPACE_TOO_SMALL = 3,/* metadata or workspace buffer smaller than the size query said */
  LI_ERR_HIP = 4,                /* a HIP runtime call failed (launch error) */
  LI_ERR_METADATA_MISMATCH = 5   /* device-side only: the metadata passed to li_forward was not
                                    built by li_metadata for this problem (see li_forward) */
} li_status;

typedef enum {
  LI_LAYOUT_BSND = 0,            /* [B, S, N, D], batch-padded */
  LI_LAYOUT_TND = 1,             /* [T, N, D], packed, with inclusive cu_seqlens */
  LI_LAYOUT_PA_BSND = 2          /* keys only: paged pool [num_blocks, block_size, 1, D] */
} li_layout;

typedef enum {
  LI_DT_BF16 = 0,
  LI_DT_FP8_E4M3 = 1,            /* OCP e4m3fn codes, needs q_descale and k_descale */
  LI_DT_FP32 = 2,                /* weights only */
  LI_DT_FP16 = 3
} li_dtype;

/*
 * Problem description (host memory, read during the call only).
 * Ranges follow the pages' constraints (lightning_indexer page, Constraints;
 * aclnnLightningIndexerV2 page, 约束说明): N of q in [1, 64], N of k = 1, head dim
 * 128, q and k of one dtype, topk in [1, 2048] or one of 3072, 4096, 5120, 6144, 7168,
 * 8192, paged block size in [1, 1024] with 32-byte-aligned blocks, and axis 0 of the
 * paged pool may be non-contiguous.
 */
typedef struct {
  int32_t batch;                 /* B >= 0                                                  */
  int32_t max_seqlen_q;          /* BSND: S1.  TND: an upper bound of every S1_b            */
  int32_t max_seqlen_k;          /* BSND: S2.  TND / PA: an upper bound of every S2_b       */
  int32_t total_q;               /* TND q: T1 (= cu_seqlens_q[B-1]); else ignored           */
  int32_t total_k;               /* TND k: T2 (= cu_seqlens_k[B-1]); else ignored           */
  int32_t num_heads_q;           /* N1 in [1, 64]                                           */
  int32_t num_heads_k;           /* N2, must be 1                                           */
  int32_t head_dim;              /* D, must be 128                                          */
  int32_t topk;                  /* [1, 2048], or 3072 .. 8192 in steps of 1024             */
  int32_t layout_q;              /* li_layout: BSND or TND                                  */
  int32_t layout_k;              /* li_layout: BSND, TND or PA_BSND                         */
  int32_t mask_mode;             /* 0 or 3                                                  */
  int32_t qk_dtype;              /* li_dtype: BF16, FP16 or FP8_E4M3 (q and k alike)        */
  int32_t w_dtype;               /* li_dtype: BF16 or FP32                                  */
  int32_t block_size;            /* PA only: [1, 1024], block_size*D*elem % 32 == 0         */
  int32_t num_blocks;            /* PA only: blocks in the pool (> 0)                       */
  int32_t max_blocks_per_seq;    /* PA only: columns of block_table (> 0)                   */
  int32_t cmp_ratio;             /* >= 1: original key positions per key of k (compressed
                                    keys); 1 = no compression                              */
  int64_t k_block_stride;        /* PA only: elements between pool blocks, >= block_size*D;
                                    0 means block_size*D (a contiguous pool)                */
} li_problem;

/* Bytes of the metadata buffer that li_metadata fills for this problem.  Host
 * only: validates the scalars, makes no HIP call. */
li_status li_metadata_size(const li_problem* p, size_t* bytes);

/* Bytes of device workspace li_forward needs (at least 256: a status block, then the
 * kernels' scratch).  Host only. */
li_status li_workspace_size(const li_problem* p, size_t* bytes);

/*
 * Builds the work list for li_forward on `stream` (one small kernel).
 *  cu_seqlens_q : int32 [B], inclusive prefix sums of query lengths; required iff
 *                 layout_q == TND, must be NULL otherwise.
 *  cu_seqlens_k : int32 [B], inclusive prefix sums of key lengths; required iff
 *                 layout_k == TND, must be NULL otherwise.
 *  seqused_k    : int32 [B], keys used per batch; required iff layout_k == PA_BSND,
 *                 must be NULL otherwise.
 *  cmp_residual_k : int32 [B], each in [0, cmp_ratio): original keys of the batch
 *                 past its last compressed key; required iff cmp_ratio > 1 and
 *                 mask_mode == 3, must be NULL otherwise (aclnnLightningIndexerV2
 *                 page, 约束说明).  Batch b then has S2_b * cmp_ratio + residual
 *                 original keys; local row i is original position
 *                 i + S2_b * cmp_ratio + residual - S1_b and sees key j when
 *                 j * cmp_ratio + cmp_ratio - 1 is at or before it.
 *  metadata     : device buffer of at least li_metadata_size bytes, 256-byte aligned.
 * The metadata stays valid for any li_forward call with the same problem and the
 * same length arrays.  li_forward changes nothing in it but two words of its
 * header, a work counter that prefill rows past 4096 keys use and leave at zero:
 * so one metadata buffer serves one li_forward at a time (calls that may overlap
 * on the device, on different streams, need buffers of their own).
 */
li_status li_metadata(const li_problem* p, const int32_t* cu_seqlens_q,
                      const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                      const int32_t* cmp_residual_k, void* metadata, size_t metadata_bytes,
                      hipStream_t stream);

/*
 * Scores every visible (query, key) pair and writes the per-token top-k.
 *  q            : BSND [B, S1, N1, 128] or TND [T1, N1, 128], contiguous, qk_dtype.
 *  k            : BSND [B, S2, 1, 128], TND [T2, 1, 128] (contiguous), or the paged
 *                 pool [num_blocks, block_size, 1, 128] whose block stride is
 *                 k_block_stride elements (rows inside a block contiguous).
 *  w            : [B, S1, N1] or [T1, N1], contiguous, w_dtype.
 *  q_descale    : fp32, one per query token ([B, S1] or [T1]); required iff fp8.
 *  k_descale    : fp32, one per key slot ([B, S2], [T2], or [num_blocks, block_size]
 *                 contiguous for the paged pool); required iff fp8.
 *  cu_seqlens_q, cu_seqlens_k, seqused_k, cmp_residual_k : as for li_metadata
 *                 (same contents).
 *  block_table  : int32 [B, max_blocks_per_seq]; required iff layout_k == PA_BSND.
 *                 Logical key s of batch b lives in row s % block_size of pool
 *                 block block_table[b][s / block_size].
 *  output_idx_offset : NULL, or int32 [B] of offsets >= 0 added to every valid
 *                 index of batch b (the -1 padding stays); index + offset must fit
 *                 int32 (aclnnLightningIndexerV2 page, 约束说明).
 *  metadata     : filled by li_metadata for this problem.  Its header holds a
 *                 fingerprint of the li_problem scalars it was built for; every kernel
 *                 compares it with the fingerprint of `p` before it reads a work item.
 *                 On a mismatch (metadata of another problem) nothing is read from the
 *                 work list: every output slot receives -1 / -inf and the status word
 *                 (below) becomes LI_ERR_METADATA_MISMATCH.  The call itself still
 *                 returns LI_OK, since the check runs on the device.
 *  workspace    : li_workspace_size bytes of device memory, 256-byte aligned; its
 *                 contents need no initialisation.  Its first int32 is the status word:
 *                 once the call has completed on `stream` it holds LI_OK or
 *                 LI_ERR_METADATA_MISMATCH.
 *  sparse_indices : int32 [B, S1, 1, topk] or [T1, 1, topk].
 *  sparse_values  : fp32, same shape, or NULL to skip values (the pages'
 *                   return_value = 0).
 * q, k, w and the descales must be 16-byte aligned.
 */
li_status li_forward(const li_problem* p, const void* q, const void* k, const void* w,
                     const float* q_descale, const float* k_descale,
                     const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                     const int32_t* seqused_k, const int32_t* cmp_residual_k,
                     const int32_t* block_table, const int32_t* output_idx_offset,
                     const void* metadata, void* workspace, size_t workspace_bytes,
                     int32_t* sparse_indices, float* sparse_values, hipStream_t stream);

/*
 * li_forward without a workspace argument, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as li_forward otherwise.  The kernels'
 * scratch is one file-scope device array of 128 MiB per GPU (allocated with the
 * library's code on that GPU and held until the process ends); the call makes no
 * hipMalloc / hipFree and allocates nothing.  The current device's copy is looked
 * up on the first call on that device (hipGetSymbolAddress), so the calling thread's
 * current device must be the one `stream` belongs to.
 *  - A problem whose li_workspace_size exceeds 128 MiB is rejected with
 *    LI_ERR_WORKSPACE_TOO_SMALL before any HIP call (use li_forward for it).
 *  - Every call on one GPU shares that GPU's array, which keeps the last call's
 *    contents: calls that overlap on one GPU (other streams or threads) race and
 *    must be serialised by the caller.  Nothing in it needs to start at zero.
 *  - The status word of li_forward lives in that array; a metadata mismatch still
 *    writes -1 / -inf into every output slot.
 */
li_status li_forward_noalloc(const li_problem* p, const void* q, const void* k, const void* w,
                             const float* q_descale, const float* k_descale,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             const int32_t* seqused_k, const int32_t* cmp_residual_k,
                             const int32_t* block_table, const int32_t* output_idx_offset,
                             const void* metadata, int32_t* sparse_indices, float* sparse_values,
                             hipStream_t stream);

/*
 * Gathers, for every query row, the key (or value) rows its top-k selected: the
 * step after the indexer, where sparse attention reads its selected keys
 * (aclnnSparseFlashAttentionGrad page, calculation formula: the selected key is
 * the gather of key by topkIndices[i] for i < selectBlockCount, each index a
 * block of selectedBlockSize tokens).  One kernel on `stream`.
 *  p            : the problem given to li_forward (layouts, lengths, topk, paged
 *                 block size); its head counts and dtype are not used.
 *  kv           : the token rows, row_bytes each (a multiple of 16; any element
 *                 type), in the key layout of p: BSND [B, S2, row], TND [T2, row], or
 *                 the paged pool [num_blocks, block_size, row] whose blocks are
 *                 kv_block_stride bytes apart (0: block_size * row_bytes).
 *  sparse_indices : int32 [rows, topk], as li_forward wrote them without an output
 *                 index offset (sequence-local positions, -1 padding).
 *  select_block : tokens per index (selectedBlockSize, >= 1): index i selects the
 *                 tokens i * select_block .. i * select_block + select_block - 1.
 *  block_table  : int32 [B, max_blocks_per_seq]; required iff layout_k == PA_BSND.
 *  metadata     : filled by li_metadata for p (checked as in li_forward: with metadata
 *                 of another problem every output row is zero bytes).
 *  out          : [rows, topk * select_block, row_bytes] bytes, 16-byte aligned.  An
 *                 index of -1, or a token at or past the sequence's key count, gives a
 *                 row of zero bytes.
 * kv must be 16-byte aligned.
 */
li_status li_gather(const li_problem* p, const void* kv, int32_t row_bytes, int64_t kv_block_stride,
                    const int32_t* sparse_indices, int32_t select_block,
                    const int32_t* block_table, const void* metadata, void* out,
                    hipStream_t stream);

/*
 * Backward of the indexer fused with its KL loss (npu_sparse_lightning_indexer_grad_kl_loss
 * page, 计算公式 items 1-4 and its parameter list).  For query token t and the keys s_j
 * that the valid entries of sparse_indices[t] select:
 *   I_j  = sum_h w[t,h] ReLU(S_h,j),  S_h,j = q_index[t,h,:] . k_index[s_j,:]
 *   p_j  = sum_g exp(scale (q[t,g,:] . k[s_j,:] + q_rope[t,g,:] . k_rope[s_j,:]) - softmax_max[t,g])
 *          / softmax_sum[t,g], normalised to sum 1 over j (the main attention's probabilities,
 *          recomputed from the statistics its forward saved, summed over the heads)
 *   loss = sum_t sum_j p_j (log p_j - log Softmax(I)_j)       (KL(p || Softmax(I)))
 *   dI   = Softmax(I) - p;  d_w[t,h] = sum_j dI_j ReLU(S_h,j);  dS_h,j = dI_j w[t,h] [S_h,j > 0]
 *   d_q_index[t,h,:] = sum_j dS_h,j k_index[s_j,:];  d_k_index[s,:] = sum over (t, j, h) with
 *          s_j = s of dS_h,j q_index[t,h,:]
 * Readings where the page is silent: the distributions run over the selected keys only
 * (entries of -1, or at or past the sequence's key count, are skipped); scale_value takes
 * the place of 1/sqrt(d); the main attention has one key head shared by its G query
 * heads, so softmax_max / softmax_sum are [rows, G] (the page's (B, N2, S1, G) with N2 = 1);
 * all outputs are fp32.
 */
typedef struct {
  int32_t batch;                 /* B >= 0                                                  */
  int32_t max_seqlen_q;          /* BSND: S1.  TND: an upper bound of every S1_b            */
  int32_t max_seqlen_k;          /* BSND: S2.  TND: an upper bound of every S2_b            */
  int32_t total_q;               /* TND: T1 (= cu_seqlens_q[B-1]); else ignored             */
  int32_t total_k;               /* TND: T2 (= cu_seqlens_k[B-1]); else ignored             */
  int32_t layout;                /* li_layout BSND or TND, the query and key sides alike    */
  int32_t num_heads;             /* G: main-attention query heads, [1, 64]                  */
  int32_t head_dim;              /* main-attention head dim: 128                            */
  int32_t rope_dim;              /* 0 (no rope inputs) or 64                                */
  int32_t num_heads_index;       /* indexer query heads, [1, 64]                            */
  int32_t head_dim_index;        /* 128                                                     */
  int32_t topk;                  /* entries per sparse_indices row, [1, 2048]               */
  int32_t dtype;                 /* li_dtype BF16 or FP16: q, k, q_rope, k_rope, q_index,
                                    k_index alike                                          */
  int32_t w_dtype;               /* li_dtype BF16 or FP32                                   */
  float scale;                   /* scale_value                                             */
} li_grad_problem;

/* Bytes of device workspace li_grad_kl needs (the per-row losses).  Host only. */
li_status li_grad_workspace_size(const li_grad_problem* p, size_t* bytes);

/*
 * Loss and gradients of the KL objective above, enqueued on `stream` (a fill kernel for
 * d_k_index, the row kernel, a reduction of the loss).  Device pointers owned by the
 * caller; the library allocates nothing.
 *  q, k         : main attention: BSND [B, S1, G, 128] / [B, S2, 1, 128], or TND [T1, G, 128] /
 *                 [T2, 1, 128]; q_rope, k_rope the same with 64 dims (NULL iff rope_dim == 0).
 *  q_index, k_index : [B, S1, Ni, 128] / [B, S2, 1, 128], or [T1, Ni, 128] / [T2, 1, 128].
 *  w            : [B, S1, Ni] or [T1, Ni], w_dtype.
 *  sparse_indices : int32 [rows, topk], sequence-local key positions (li_forward's output
 *                 without an index offset); -1 entries are skipped.
 *  softmax_max, softmax_sum : fp32 [rows, G].
 *  cu_seqlens_q, cu_seqlens_k : int32 [B] inclusive prefix sums; required iff TND.
 *  workspace    : li_grad_workspace_size bytes, 16-byte aligned.
 *  d_q_index    : fp32 [rows, Ni, 128];  d_w : fp32 [rows, Ni];  d_k_index : fp32 [keys, 128]
 *                 (fully overwritten; d_k_index is summed with fp32 atomics, so its low bits
 *                 may differ from run to run);  loss : fp32 [1], the sum over the rows (the
 *                 per-row losses stay in the workspace as fp32 [rows]).
 * Tensors of 16-bit elements and w must be 16-byte aligned.
 */
li_status li_grad_kl(const li_grad_problem* p, const void* q, const void* k, const void* q_rope,
                     const void* k_rope, const void* q_index, const void* k_index, const void* w,
                     const int32_t* sparse_indices, const float* softmax_max,
                     const float* softmax_sum, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_k, void* workspace, size_t workspace_bytes,
                     float* d_q_index, float* d_k_index, float* d_w, float* loss,
                     hipStream_t stream);

/* Static, human-readable name of a status code. */
const char* li_status_str(li_status s);

#ifdef __cplusplus
}
#endif
#endif /* LI_H */
