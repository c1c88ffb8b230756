// Host side of the C ABI (include/li.h): argument validation, sizing, the
// launch plan, and the kernel launches.  No device memory is allocated and the
// host never waits for the device here.
#include <string.h>

#include <algorithm>
#include <mutex>

#include <hip/hip_runtime.h>

#include "li.h"
#include "li_internal.h"

using namespace li;

namespace {

inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

int elem_bytes(int dt) { return dt == LI_DT_FP8_E4M3 ? 1 : (dt == LI_DT_FP32 ? 4 : 2); }

// Scalar checks (no pointers, no HIP).  Ranges from the pages' constraint lists
// (lightning_indexer page, Constraints; aclnnLightningIndexerV2 page, 约束说明).
li_status validate_scalars(const li_problem* p) {
  if (!p) return LI_ERR_INVALID_ARGUMENT;
  if (p->batch < 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0) return LI_ERR_INVALID_ARGUMENT;
  if (p->num_heads_q < 1 || p->num_heads_q > kMaxHeads) return LI_ERR_INVALID_ARGUMENT;
  if (p->num_heads_k != 1) return LI_ERR_INVALID_ARGUMENT;
  if (p->head_dim != kHeadDim) return LI_ERR_INVALID_ARGUMENT;
  if (p->topk < 1) return LI_ERR_INVALID_ARGUMENT;
  // [1, 2048], then 3072 .. 8192 in steps of 1024
  if (p->topk > kMaxTopk && (p->topk > kMaxTopkLarge || p->topk % 1024 != 0))
    return LI_ERR_INVALID_ARGUMENT;
  if (p->layout_q != LI_LAYOUT_BSND && p->layout_q != LI_LAYOUT_TND) return LI_ERR_INVALID_ARGUMENT;
  if (p->layout_k != LI_LAYOUT_BSND && p->layout_k != LI_LAYOUT_TND &&
      p->layout_k != LI_LAYOUT_PA_BSND)
    return LI_ERR_INVALID_ARGUMENT;
  if (p->mask_mode != 0 && p->mask_mode != 3) return LI_ERR_INVALID_ARGUMENT;
  if (p->qk_dtype != LI_DT_BF16 && p->qk_dtype != LI_DT_FP16 && p->qk_dtype != LI_DT_FP8_E4M3)
    return LI_ERR_INVALID_ARGUMENT;
  if (p->w_dtype != LI_DT_BF16 && p->w_dtype != LI_DT_FP32) return LI_ERR_INVALID_ARGUMENT;
  if (p->cmp_ratio < 1) return LI_ERR_INVALID_ARGUMENT;
  if (p->layout_q == LI_LAYOUT_TND && p->total_q < 0) return LI_ERR_INVALID_ARGUMENT;
  if (p->layout_k == LI_LAYOUT_TND && p->total_k < 0) return LI_ERR_INVALID_ARGUMENT;
  if (p->layout_k == LI_LAYOUT_PA_BSND) {
    if (p->block_size < 1 || p->block_size > 1024) return LI_ERR_INVALID_ARGUMENT;
    if (((int64_t)p->block_size * kHeadDim * elem_bytes(p->qk_dtype)) % 32 != 0)
      return LI_ERR_INVALID_ARGUMENT;
    if (p->num_blocks < 1 || p->max_blocks_per_seq < 1) return LI_ERR_INVALID_ARGUMENT;
    const int64_t contig = (int64_t)p->block_size * kHeadDim;
    if (p->k_block_stride != 0 && p->k_block_stride < contig) return LI_ERR_INVALID_ARGUMENT;
    if ((p->k_block_stride * elem_bytes(p->qk_dtype)) % 16 != 0) return LI_ERR_INVALID_ARGUMENT;
    if ((int64_t)p->max_seqlen_k > (int64_t)p->max_blocks_per_seq * p->block_size)
      return LI_ERR_INVALID_ARGUMENT;
  }
  // 32-bit token offsets inside the kernels
  const int64_t rows = p->layout_q == LI_LAYOUT_TND ? p->total_q
                                                    : (int64_t)p->batch * p->max_seqlen_q;
  const int64_t keys = p->layout_k == LI_LAYOUT_TND ? p->total_k
                                                    : (int64_t)p->batch * p->max_seqlen_k;
  if (rows > INT32_MAX || keys > INT32_MAX) return LI_ERR_UNSUPPORTED;
  return LI_OK;
}

int64_t query_rows(const li_problem* p) {
  return p->layout_q == LI_LAYOUT_TND ? p->total_q : (int64_t)p->batch * p->max_seqlen_q;
}

// Decode mode: a few query rows per batch and a bounded dense score workspace.
bool use_decode(const li_problem* p) {
  if (p->max_seqlen_q > kDecodeMaxRows || p->max_seqlen_k <= 0) return false;
  const int64_t ws = (int64_t)p->batch * p->max_seqlen_q * align_up(p->max_seqlen_k, 64) * 4;
  return ws <= (int64_t(1) << 30);
}

int64_t prefill_items(const li_problem* p, int rows) {
  if (p->layout_q == LI_LAYOUT_TND)
    return std::min<int64_t>(cdiv64(p->total_q, rows) + p->batch,
                             (int64_t)p->batch * cdiv64(p->max_seqlen_q, rows));
  return (int64_t)p->batch * cdiv64(p->max_seqlen_q, rows);
}

li_status make_plan(const li_problem* p, Plan* pl) {
  li_status st = validate_scalars(p);
  if (st != LI_OK) return st;
  memset(pl, 0, sizeof(*pl));
  const int B = p->batch;
  pl->mblocks = p->num_heads_q <= 32 ? 1 : 2;
  const size_t rb = (size_t)kHeadDim * elem_bytes(p->qk_dtype);     // bytes per key row
  const int64_t dcap = (int64_t)align_up(std::max(p->max_seqlen_k, 1), 64);
  // two 32-key K tiles and, for fp8, the descale slots (4 x 32 floats), or the
  // per-wave select scratch, whichever is larger; then the score rows
  const size_t tiles = 2 * (size_t)kPipeKeys * rb + (p->qk_dtype == LI_DT_FP8_E4M3 ? 4 * 32 * 4 : 0);
  const size_t dense_r0 = std::max(tiles, (size_t)kDenseWaves * kDenseScratch);
  // before the score loop each wave stages a 32-head block of its query in the
  // same space
  const size_t q_stage = (size_t)kDenseWaves * 32 * rb;
  const size_t dense_lds = std::max(dense_r0 + (size_t)kDenseWaves * dcap * 4, q_stage);
  int64_t items;
  if (use_decode(p)) {
    pl->mode = kModeDecode;
    pl->chunk = kTileKeys;                // minimum segment; the device picks the real one
    // segments <= target + rows, target <= kDecodeSegments + 2 * rows; padded
    // to whole rounds of 8 workgroups
    items = align_up(3 * (int64_t)B * p->max_seqlen_q + kDecodeSegments, 8 * kDecodeWaves);
    pl->ws_row_stride = (int64_t)align_up(p->max_seqlen_k, 64);
    // then the (min, max) of each segment (at least kTileKeys keys long)
    pl->seg_mm_stride = (int32_t)cdiv64(std::max(p->max_seqlen_k, 1), kTileKeys);
    pl->ws_bytes = (size_t)B * p->max_seqlen_q * ((size_t)pl->ws_row_stride * 4 + (size_t)pl->seg_mm_stride * 8);
    pl->lds_select = select_shared_bytes();
  } else if (dense_lds <= kLdsBudget / 2) {
    // two workgroups per CU
    pl->mode = kModeDense;
    pl->rows_per_item = kDenseWaves;
    pl->dcap = (int32_t)dcap;
    pl->lds_prefill = dense_lds;
    items = prefill_items(p, kDenseWaves);
  } else if (p->max_seqlen_k <= kGlobalRowKeys) {
    // rows too long for LDS: the same kernel with each row in a workspace row,
    // one per wave of a fixed grid of resident workgroups (two per CU) walking
    // the work list
    pl->mode = kModeDenseGlobal;
    pl->rows_per_item = kDenseWaves;
    items = prefill_items(p, kDenseWaves);
    pl->grid = (int32_t)std::min<int64_t>(items, kDenseSlots);
    pl->ws_row_stride = dcap;
    pl->ws_bytes = (size_t)pl->grid * kDenseWaves * dcap * 4;
    pl->lds_prefill = std::max(std::max(tiles, (size_t)kDenseWaves * kWideScratch), q_stage);
  } else {
    // longer rows: the same grid; each row keeps its running top-k in its
    // output slots and a candidate list in LDS (after the K tiles, the descale
    // slots, the per-wave merge scratch and one int flag per wave)
    pl->mode = kModeDenseList;
    pl->rows_per_item = kDenseWaves;
    items = prefill_items(p, kDenseWaves);
    pl->grid = (int32_t)std::min<int64_t>(items, kDenseSlots);
    const size_t fixed = tiles + (size_t)kDenseWaves * kListScratch + 16;
    const int cap = (int)((kLdsBudget / 2 - fixed) / ((size_t)kDenseWaves * 8) / 64 * 64);
    if (cap < 2 * kListRoom) return LI_ERR_UNSUPPORTED;
    pl->cap = cap;
    pl->lds_prefill = std::max(fixed + (size_t)kDenseWaves * cap * 8, q_stage);
    // the running top-k's values when sparse_values is NULL: topk floats per resident wave
    pl->ws_bytes = (size_t)pl->grid * kDenseWaves * p->topk * 4;
  }
  // the status block ahead of the kernels' scratch
  pl->ws_bytes += kStatusBytes;
  if (items > INT32_MAX / 16) return LI_ERR_UNSUPPORTED;
  pl->max_items = (int32_t)items;
  pl->off_batch = sizeof(MetaHeader);
  pl->off_counts = align_up(pl->off_batch + (size_t)B * 16, 16);
  pl->off_starts = align_up(pl->off_counts + (size_t)B * 4, 16);
  pl->off_items = align_up(pl->off_starts + (size_t)B * 4, 16);
  pl->meta_bytes = pl->off_items + (size_t)pl->max_items * 16;
  if (pl->meta_bytes > (size_t)INT32_MAX) return LI_ERR_UNSUPPORTED;
  return LI_OK;
}

bool aligned(const void* ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

// FNV-1a over every scalar of the problem: li_metadata stores it in the
// metadata header, and each kernel of li_forward / li_gather compares it with
// the fingerprint of its own problem before it reads an item.
uint32_t fingerprint(const li_problem* p) {
  uint32_t h = 2166136261u;
  auto mix = [&](int64_t v) {
    for (int i = 0; i < 8; ++i) {
      h ^= (uint32_t)((uint64_t)v >> (8 * i)) & 0xFFu;
      h *= 16777619u;
    }
  };
  const int64_t f[] = {p->batch, p->max_seqlen_q, p->max_seqlen_k, p->total_q, p->total_k,
                       p->num_heads_q, p->num_heads_k, p->head_dim, p->topk, p->layout_q,
                       p->layout_k, p->mask_mode, p->qk_dtype, p->w_dtype, p->block_size,
                       p->num_blocks, p->max_blocks_per_seq, p->cmp_ratio, p->k_block_stride};
  for (int64_t v : f) mix(v);
  return h;
}

// Pointer presence rules shared by li_metadata and li_forward
// (aclnnLightningIndexerV2 page, 约束说明: cu_seqlens only with TND layouts,
// seqused_k required with, and only with, the paged key layout).
li_status validate_lengths(const li_problem* p, const int32_t* cu_q, const int32_t* cu_k,
                           const int32_t* seqused_k, const int32_t* cmp_res) {
  // the compression residuals come with, and only with, compressed keys under mask 3
  if ((p->cmp_ratio > 1 && p->mask_mode == 3) != (cmp_res != nullptr))
    return LI_ERR_INVALID_ARGUMENT;
  if ((p->layout_q == LI_LAYOUT_TND) != (cu_q != nullptr)) return LI_ERR_INVALID_ARGUMENT;
  if ((p->layout_k == LI_LAYOUT_TND) != (cu_k != nullptr)) return LI_ERR_INVALID_ARGUMENT;
  if ((p->layout_k == LI_LAYOUT_PA_BSND) != (seqused_k != nullptr)) return LI_ERR_INVALID_ARGUMENT;
  return LI_OK;
}

KArgs base_args(const li_problem* p, const Plan& pl, void* metadata) {
  KArgs a;
  memset(&a, 0, sizeof(a));
  a.meta = static_cast<unsigned char*>(metadata);
  a.batch = p->batch;
  a.s1max = p->max_seqlen_q;
  a.s2max = p->max_seqlen_k;
  a.n1 = p->num_heads_q;
  a.topk = p->topk;
  a.layout_q = p->layout_q;
  a.layout_k = p->layout_k;
  a.mask_mode = p->mask_mode;
  a.block_size = p->block_size;
  a.max_blocks_per_seq = p->max_blocks_per_seq;
  const int64_t kbs = p->k_block_stride ? p->k_block_stride : (int64_t)p->block_size * kHeadDim;
  a.k_block_stride_bytes = kbs * elem_bytes(p->qk_dtype);
  a.cmp_ratio = p->cmp_ratio;
  a.block_shift = -1;
  if (p->block_size > 0 && (p->block_size & (p->block_size - 1)) == 0)
    a.block_shift = __builtin_ctz((unsigned)p->block_size);
  a.cap = pl.cap;
  a.dcap = pl.dcap;
  a.rows_per_item = pl.rows_per_item;
  a.chunk = pl.chunk;
  a.max_items = pl.max_items;
  a.ws_row_stride = pl.ws_row_stride;
  a.seg_mm_stride = pl.seg_mm_stride;
  a.off_batch = (int32_t)pl.off_batch;
  a.off_counts = (int32_t)pl.off_counts;
  a.off_starts = (int32_t)pl.off_starts;
  a.off_items = (int32_t)pl.off_items;
  a.fingerprint = fingerprint(p);
  a.rows = (int32_t)query_rows(p);
  return a;
}

}  // namespace

extern "C" {

li_status li_metadata_size(const li_problem* p, size_t* bytes) {
  if (!bytes) return LI_ERR_INVALID_ARGUMENT;
  Plan pl;
  li_status st = make_plan(p, &pl);
  if (st != LI_OK) return st;
  *bytes = pl.meta_bytes;
  return LI_OK;
}

li_status li_workspace_size(const li_problem* p, size_t* bytes) {
  if (!bytes) return LI_ERR_INVALID_ARGUMENT;
  Plan pl;
  li_status st = make_plan(p, &pl);
  if (st != LI_OK) return st;
  *bytes = pl.ws_bytes;
  return LI_OK;
}

li_status li_metadata(const li_problem* p, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                      const int32_t* seqused_k, const int32_t* cmp_residual_k, void* metadata,
                      size_t metadata_bytes, hipStream_t stream) {
  Plan pl;
  li_status st = make_plan(p, &pl);
  if (st != LI_OK) return st;
  st = validate_lengths(p, cu_seqlens_q, cu_seqlens_k, seqused_k, cmp_residual_k);
  if (st != LI_OK) return st;
  if (!metadata || !aligned(metadata, 16)) return LI_ERR_INVALID_ARGUMENT;
  if (metadata_bytes < pl.meta_bytes) return LI_ERR_WORKSPACE_TOO_SMALL;
  if (query_rows(p) == 0) return LI_OK;
  KArgs a = base_args(p, pl, metadata);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.seqused_k = seqused_k;
  a.cmp_res = cmp_residual_k;
  return launch_metadata(a, pl.mode, stream) == hipSuccess ? LI_OK : LI_ERR_HIP;
}

}  // extern "C"

namespace {

// Every check of li_forward that needs neither the workspace nor device data.
li_status forward_checks(const li_problem* p, Plan* pl, const void* q, const void* k,
                         const void* w, const float* q_descale, const float* k_descale,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         const int32_t* seqused_k, const int32_t* cmp_residual_k,
                         const int32_t* block_table, const void* metadata,
                         const int32_t* sparse_indices) {
  li_status st = make_plan(p, pl);
  if (st != LI_OK) return st;
  st = validate_lengths(p, cu_seqlens_q, cu_seqlens_k, seqused_k, cmp_residual_k);
  if (st != LI_OK) return st;
  if ((p->layout_k == LI_LAYOUT_PA_BSND) != (block_table != nullptr)) return LI_ERR_INVALID_ARGUMENT;
  const bool fp8 = p->qk_dtype == LI_DT_FP8_E4M3;
  if (fp8 != (q_descale != nullptr) || fp8 != (k_descale != nullptr)) return LI_ERR_INVALID_ARGUMENT;
  if (!q || !k || !w || !metadata || !sparse_indices) return LI_ERR_INVALID_ARGUMENT;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(w, 16) || !aligned(metadata, 16))
    return LI_ERR_INVALID_ARGUMENT;
  if (fp8 && (!aligned(q_descale, 4) || !aligned(k_descale, 4))) return LI_ERR_INVALID_ARGUMENT;
  return LI_OK;
}

// The launches of li_forward once every argument has been checked; `workspace`
// holds pl.ws_bytes (status block first).
li_status forward_launch(const li_problem* p, const Plan& pl, const void* q, const void* k,
                         const void* w, const float* q_descale, const float* k_descale,
                         const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                         const int32_t* seqused_k, const int32_t* cmp_residual_k,
                         const int32_t* block_table, const int32_t* output_idx_offset,
                         const void* metadata, void* workspace, int32_t* sparse_indices,
                         float* sparse_values, hipStream_t stream) {
  KArgs a = base_args(p, pl, const_cast<void*>(metadata));
  a.q = q;
  a.k = k;
  a.w = w;
  a.q_descale = q_descale;
  a.k_descale = k_descale;
  a.block_table = block_table;
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.seqused_k = seqused_k;
  a.cmp_res = cmp_residual_k;
  a.idx_off = output_idx_offset;
  a.status = static_cast<int32_t*>(workspace);
  a.ws = reinterpret_cast<float*>(static_cast<unsigned char*>(workspace) + kStatusBytes);
  if (pl.mode == kModeDecode)
    a.seg_mm = a.ws + (size_t)p->batch * p->max_seqlen_q * pl.ws_row_stride;
  a.out_idx = sparse_indices;
  a.out_val = sparse_values;
  const int qk = p->qk_dtype, wt = p->w_dtype;
  // paged blocks holding whole 32-key tiles let a tile be addressed by one lookup
  const int kl = p->layout_k != LI_LAYOUT_PA_BSND ? KL_CONTIG
                 : (p->block_size % 32 == 0 ? KL_PAGED_TILE : KL_PAGED);
  hipError_t e;
  if (pl.mode != kModeDecode) {
    const int grid = pl.mode == kModeDense ? pl.max_items : pl.grid;
    e = launch_prefill(a, pl.mode, qk, wt, pl.mblocks, kl, grid, pl.lds_prefill, stream);
  } else {
    e = launch_decode(a, qk, wt, pl.mblocks, kl,
                      (int)cdiv64(pl.max_items, kDecodeWaves), stream);
    if (e == hipSuccess)
      e = launch_select(a, p->batch * p->max_seqlen_q, pl.lds_select, stream);
  }
  return e == hipSuccess ? LI_OK : LI_ERR_HIP;
}

}  // namespace

// ---- the no-allocation entry point ------------------------------------------
// Scratch of li_forward_noalloc: one array per GPU, held until the process ends.
// In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // per device: the address of `scratch` there

// The current device's copy of `scratch` (looked up on the first call per device).
li_status device_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return LI_ERR_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return LI_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return LI_OK;
}

}  // namespace

extern "C" {

li_status li_forward(const li_problem* p, const void* q, const void* k, const void* w,
                     const float* q_descale, const float* k_descale, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_k, const int32_t* seqused_k,
                     const int32_t* cmp_residual_k, const int32_t* block_table,
                     const int32_t* output_idx_offset, const void* metadata, void* workspace,
                     size_t workspace_bytes, int32_t* sparse_indices, float* sparse_values,
                     hipStream_t stream) {
  Plan pl;
  li_status st = forward_checks(p, &pl, q, k, w, q_descale, k_descale, cu_seqlens_q, cu_seqlens_k,
                                seqused_k, cmp_residual_k, block_table, metadata, sparse_indices);
  if (st != LI_OK) return st;
  if (workspace_bytes < pl.ws_bytes) return LI_ERR_WORKSPACE_TOO_SMALL;
  if (pl.ws_bytes > 0 && (!workspace || !aligned(workspace, 16))) return LI_ERR_INVALID_ARGUMENT;
  if (query_rows(p) == 0) return LI_OK;
  return forward_launch(p, pl, q, k, w, q_descale, k_descale, cu_seqlens_q, cu_seqlens_k,
                        seqused_k, cmp_residual_k, block_table, output_idx_offset, metadata,
                        workspace, sparse_indices, sparse_values, stream);
}

li_status li_forward_noalloc(const li_problem* p, const void* q, const void* k, const void* w,
                             const float* q_descale, const float* k_descale,
                             const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                             const int32_t* seqused_k, const int32_t* cmp_residual_k,
                             const int32_t* block_table, const int32_t* output_idx_offset,
                             const void* metadata, int32_t* sparse_indices, float* sparse_values,
                             hipStream_t stream) {
  Plan pl;
  li_status st = forward_checks(p, &pl, q, k, w, q_descale, k_descale, cu_seqlens_q, cu_seqlens_k,
                                seqused_k, cmp_residual_k, block_table, metadata, sparse_indices);
  if (st != LI_OK) return st;
  if (pl.ws_bytes > kNoAllocScratchBytes) return LI_ERR_WORKSPACE_TOO_SMALL;
  if (query_rows(p) == 0) return LI_OK;
  void* ws = nullptr;
  st = device_scratch(&ws);
  if (st != LI_OK) return st;
  return forward_launch(p, pl, q, k, w, q_descale, k_descale, cu_seqlens_q, cu_seqlens_k,
                        seqused_k, cmp_residual_k, block_table, output_idx_offset, metadata, ws,
                        sparse_indices, sparse_values, stream);
}

li_status li_gather(const li_problem* p, const void* kv, int32_t row_bytes, int64_t kv_block_stride,
                    const int32_t* sparse_indices, int32_t select_block,
                    const int32_t* block_table, const void* metadata, void* out,
                    hipStream_t stream) {
  Plan pl;
  li_status st = make_plan(p, &pl);
  if (st != LI_OK) return st;
  if (row_bytes <= 0 || row_bytes % 16 != 0 || select_block < 1) return LI_ERR_INVALID_ARGUMENT;
  if ((p->layout_k == LI_LAYOUT_PA_BSND) != (block_table != nullptr)) return LI_ERR_INVALID_ARGUMENT;
  if (!kv || !sparse_indices || !metadata || !out) return LI_ERR_INVALID_ARGUMENT;
  if (!aligned(kv, 16) || !aligned(out, 16) || !aligned(sparse_indices, 4) || !aligned(metadata, 16))
    return LI_ERR_INVALID_ARGUMENT;
  int64_t stride = 0;
  if (p->layout_k == LI_LAYOUT_PA_BSND) {
    stride = kv_block_stride ? kv_block_stride : (int64_t)p->block_size * row_bytes;
    if (stride < (int64_t)p->block_size * row_bytes || stride % 16 != 0) return LI_ERR_INVALID_ARGUMENT;
  }
  const int64_t rows = query_rows(p);
  if (rows == 0) return LI_OK;
  const int64_t per_row = (int64_t)p->topk * select_block;
  if (per_row > INT32_MAX / 16 || rows * cdiv64(per_row, kGatherRows) > INT32_MAX)
    return LI_ERR_UNSUPPORTED;
  KArgs a = base_args(p, pl, const_cast<void*>(metadata));
  a.k = kv;
  a.block_table = block_table;
  a.k_block_stride_bytes = stride;
  const GatherArgs g{sparse_indices, static_cast<unsigned char*>(out), row_bytes, select_block};
  return launch_gather(a, g, rows, stream) == hipSuccess ? LI_OK : LI_ERR_HIP;
}

// ---- backward fused with the KL loss -------------------------------------------

static li_status grad_validate(const li_grad_problem* p) {
  if (!p) return LI_ERR_INVALID_ARGUMENT;
  if (p->batch < 0 || p->max_seqlen_q < 0 || p->max_seqlen_k < 0) return LI_ERR_INVALID_ARGUMENT;
  if (p->layout != LI_LAYOUT_BSND && p->layout != LI_LAYOUT_TND) return LI_ERR_INVALID_ARGUMENT;
  if (p->layout == LI_LAYOUT_TND && (p->total_q < 0 || p->total_k < 0))
    return LI_ERR_INVALID_ARGUMENT;
  if (p->num_heads < 1 || p->num_heads > kMaxHeads) return LI_ERR_INVALID_ARGUMENT;
  if (p->num_heads_index < 1 || p->num_heads_index > kMaxHeads) return LI_ERR_INVALID_ARGUMENT;
  if (p->head_dim != kHeadDim || p->head_dim_index != kHeadDim) return LI_ERR_INVALID_ARGUMENT;
  if (p->rope_dim != 0 && p->rope_dim != 64) return LI_ERR_INVALID_ARGUMENT;
  if (p->topk < 1 || p->topk > kMaxTopk) return LI_ERR_INVALID_ARGUMENT;
  if (p->dtype != LI_DT_BF16 && p->dtype != LI_DT_FP16) return LI_ERR_INVALID_ARGUMENT;
  if (p->w_dtype != LI_DT_BF16 && p->w_dtype != LI_DT_FP32) return LI_ERR_INVALID_ARGUMENT;
  if (!(p->scale == p->scale)) return LI_ERR_INVALID_ARGUMENT;
  const int64_t rows = p->layout == LI_LAYOUT_TND ? p->total_q : (int64_t)p->batch * p->max_seqlen_q;
  const int64_t keys = p->layout == LI_LAYOUT_TND ? p->total_k : (int64_t)p->batch * p->max_seqlen_k;
  if (rows > INT32_MAX / 2 || keys * kHeadDim > INT32_MAX * (int64_t)64) return LI_ERR_UNSUPPORTED;
  return LI_OK;
}

static int64_t grad_rows(const li_grad_problem* p) {
  return p->layout == LI_LAYOUT_TND ? p->total_q : (int64_t)p->batch * p->max_seqlen_q;
}

static int64_t grad_keys(const li_grad_problem* p) {
  return p->layout == LI_LAYOUT_TND ? p->total_k : (int64_t)p->batch * p->max_seqlen_k;
}

li_status li_grad_workspace_size(const li_grad_problem* p, size_t* bytes) {
  if (!bytes) return LI_ERR_INVALID_ARGUMENT;
  li_status st = grad_validate(p);
  if (st != LI_OK) return st;
  *bytes = align_up((size_t)grad_rows(p) * 4, 256) + 256;
  return LI_OK;
}

li_status li_grad_kl(const li_grad_problem* p, const void* q, const void* k, const void* q_rope,
                     const void* k_rope, const void* q_index, const void* k_index, const void* w,
                     const int32_t* sparse_indices, const float* softmax_max,
                     const float* softmax_sum, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_k, void* workspace, size_t workspace_bytes,
                     float* d_q_index, float* d_k_index, float* d_w, float* loss,
                     hipStream_t stream) {
  li_status st = grad_validate(p);
  if (st != LI_OK) return st;
  size_t need = 0;
  li_grad_workspace_size(p, &need);
  const bool tnd = p->layout == LI_LAYOUT_TND;
  if (tnd != (cu_seqlens_q != nullptr) || tnd != (cu_seqlens_k != nullptr))
    return LI_ERR_INVALID_ARGUMENT;
  if ((p->rope_dim > 0) != (q_rope != nullptr) || (p->rope_dim > 0) != (k_rope != nullptr))
    return LI_ERR_INVALID_ARGUMENT;
  if (!q || !k || !q_index || !k_index || !w || !sparse_indices || !softmax_max || !softmax_sum ||
      !workspace || !d_q_index || !d_k_index || !d_w || !loss)
    return LI_ERR_INVALID_ARGUMENT;
  for (const void* ptr : {q, k, q_index, k_index, w})
    if (!aligned(ptr, 16)) return LI_ERR_INVALID_ARGUMENT;
  if (p->rope_dim > 0 && (!aligned(q_rope, 16) || !aligned(k_rope, 16))) return LI_ERR_INVALID_ARGUMENT;
  if (!aligned(workspace, 16) || !aligned(sparse_indices, 4) || !aligned(softmax_max, 4) ||
      !aligned(softmax_sum, 4) || !aligned(d_q_index, 4) || !aligned(d_k_index, 4) ||
      !aligned(d_w, 4) || !aligned(loss, 4))
    return LI_ERR_INVALID_ARGUMENT;
  if (workspace_bytes < need) return LI_ERR_WORKSPACE_TOO_SMALL;
  GradArgs g;
  memset(&g, 0, sizeof(g));
  g.q = q;
  g.k = k;
  g.q_rope = q_rope;
  g.k_rope = k_rope;
  g.qi = q_index;
  g.ki = k_index;
  g.w = w;
  g.sel = sparse_indices;
  g.smax = softmax_max;
  g.ssum = softmax_sum;
  g.cu_q = cu_seqlens_q;
  g.cu_k = cu_seqlens_k;
  g.d_qi = d_q_index;
  g.d_ki = d_k_index;
  g.d_w = d_w;
  g.loss = loss;
  g.loss_rows = static_cast<float*>(workspace);
  g.keys = grad_keys(p);
  g.rows = (int32_t)grad_rows(p);
  g.batch = p->batch;
  g.s1 = p->max_seqlen_q;
  g.s2 = p->max_seqlen_k;
  g.layout = p->layout;
  g.G = p->num_heads;
  g.Ni = p->num_heads_index;
  g.topk = p->topk;
  g.topk_pad = (int32_t)align_up(p->topk, 32);
  g.scale = p->scale;
  return launch_grad(g, p->dtype, p->w_dtype, p->rope_dim > 0, stream) == hipSuccess ? LI_OK
                                                                                     : LI_ERR_HIP;
}

const char* li_status_str(li_status s) {
  switch (s) {
    case LI_OK: return "LI_OK";
    case LI_ERR_INVALID_ARGUMENT: return "LI_ERR_INVALID_ARGUMENT";
    case LI_ERR_UNSUPPORTED: return "LI_ERR_UNSUPPORTED";
    case LI_ERR_WORKSPACE_TOO_SMALL: return "LI_ERR_WORKSPACE_TOO_SMALL";
    case LI_ERR_HIP: return "LI_ERR_HIP";
    case LI_ERR_METADATA_MISMATCH: return "LI_ERR_METADATA_MISMATCH";
    default: return "LI_UNKNOWN_STATUS";
  }
}

}  // extern "C"
