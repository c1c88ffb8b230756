// Gather of the key (or value) rows that the indexer selected, for the sparse
// attention that follows it (aclnnSparseFlashAttentionGrad page, calculation
// formula: the selected key is the gather of key by topkIndices[i] for
// i < selectBlockCount, each index a block of selectedBlockSize tokens).
//
// An HBM copy: each workgroup moves kGatherRows selected rows of one query row,
// 16 bytes per lane and kGatherUnroll loads in flight per lane, reading each
// token row where the key layout puts it (BSND, TND, or the paged pool through
// block_table) and writing the output densely.  An index of -1, or a token at
// or past the sequence's key count, gives a zero row.
#include "li_common_kernels.h"

namespace li {

namespace {

constexpr int kGatherThreads = 256;
constexpr int kGatherUnroll = 8;

// query row r -> (batch, local row): BSND rows are b * S1 + i; TND rows follow
// the batch table's query offsets (binary search)
__device__ inline int row_batch(const KArgs& a, int r) {
  if (a.layout_q != L_TND) return r / a.s1max;
  int lo = 0, hi = a.batch - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (batch_rec(a, mid).x <= r) lo = mid; else hi = mid - 1;
  }
  return lo;
}

__global__ __launch_bounds__(kGatherThreads) void gather_kernel(KArgs a, GatherArgs g) {
  const int per_row = a.topk * g.sel;                      // selected rows per query row
  const int slices = (per_row + kGatherRows - 1) / kGatherRows;
  const int r = blockIdx.x / slices;
  const int j0 = (blockIdx.x - r * slices) * kGatherRows;
  const int nj = min(kGatherRows, per_row - j0);
  if (!meta_matches(a)) {
    // metadata of another problem: this workgroup's rows come out as zeros
    unsigned char* o = g.out + ((int64_t)r * per_row + j0) * g.row_bytes;
    for (int e = threadIdx.x; e < nj * (g.row_bytes >> 4); e += kGatherThreads)
      reinterpret_cast<i32x4*>(o)[e] = i32x4{0, 0, 0, 0};
    return;
  }
  const int b = row_batch(a, r);
  const int4 br = batch_rec(a, b);                         // q_off, s1, k_off, s2
  const int chunks = g.row_bytes >> 4;                     // 16-byte chunks per row
  const int total = nj * chunks;
  const int32_t* idx = g.idx + (int64_t)r * a.topk;
  unsigned char* out = g.out + ((int64_t)r * per_row + j0) * g.row_bytes;
  const unsigned char* kv = reinterpret_cast<const unsigned char*>(a.k);

  for (int e0 = threadIdx.x; e0 < total; e0 += kGatherThreads * kGatherUnroll) {
    i32x4 v[kGatherUnroll];
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int e = e0 + u * kGatherThreads;
      v[u] = i32x4{0, 0, 0, 0};
      if (e < total) {
        const int j = j0 + e / chunks, c = e - (e / chunks) * chunks;
        const int sel = idx[j / g.sel];
        // in 64 bits: an index far out of range must not wrap into the row
        const int64_t s64 = (int64_t)sel * g.sel + (j - (j / g.sel) * g.sel);
        if (sel >= 0 && s64 < br.w) {
          const int s = (int)s64;
          const unsigned char* src;
          if (a.layout_k == L_PA) {
            int blk, slot;
            paged_slot(a, b, s, blk, slot);
            src = kv + (int64_t)blk * a.k_block_stride_bytes + (int64_t)slot * g.row_bytes;
          } else {
            src = kv + ((int64_t)br.z + s) * g.row_bytes;
          }
          v[u] = *reinterpret_cast<const i32x4*>(src + c * 16);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kGatherUnroll; ++u) {
      const int e = e0 + u * kGatherThreads;
      if (e < total) {
        const int j = e / chunks, c = e - j * chunks;
        *reinterpret_cast<i32x4*>(out + (int64_t)j * g.row_bytes + c * 16) = v[u];
      }
    }
  }
}

}  // namespace

hipError_t launch_gather(const KArgs& a, const GatherArgs& g, int64_t rows, hipStream_t s) {
  const int64_t per_row = (int64_t)a.topk * g.sel;
  const int64_t grid = rows * ((per_row + kGatherRows - 1) / kGatherRows);
  hipLaunchKernelGGL(gather_kernel, dim3((unsigned)grid), dim3(kGatherThreads), 0, s, a, g);
  return hipGetLastError();
}

}  // namespace li
