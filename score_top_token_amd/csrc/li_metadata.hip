// Work-list builder (the lightning_indexer page's "lightning_indexer_metadata":
// a task list that tells each core which batch and which query / key block range
// to process, for load balancing).  One workgroup reads the per-batch lengths
// (inclusive cu_seqlens for TND, seqused_k for the paged layout, the fixed BSND
// dimensions otherwise) and writes
//   - a batch table {q token offset, S1_b, k token offset, S2_b},
//   - prefill modes: one item per block of `rows_per_item` query rows, ordered so
//     that the costliest blocks (the last rows of each sequence under right-down
//     causal masking) are dispatched first, round-robin over the batches;
//   - decode mode: the visible keys of every query row cut into segments of equal
//     length (about kDecodeSegments segments in total), one item per segment.
// The result depends only on the lengths (deterministic) and is produced on the
// device, so the call never synchronises with the host.
#include "li_common_kernels.h"

namespace li {

namespace {

constexpr int kMetaThreads = 1024;
constexpr int kRoundRobinMaxBatch = 256;

__device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

__global__ __launch_bounds__(kMetaThreads) void metadata_kernel(KArgs a, int mode) {
  __shared__ int s_counts[kRoundRobinMaxBatch];
  __shared__ int s_part[kMetaThreads / 64];
  __shared__ long long s_vis[kMetaThreads / 64];
  __shared__ long long s_rows[kMetaThreads / 64];
  __shared__ int s_total, s_chunk;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int B = a.batch;
  MetaHeader* hdr = reinterpret_cast<MetaHeader*>(a.meta);
  int4* bt = reinterpret_cast<int4*>(a.meta + a.off_batch);
  int* counts = reinterpret_cast<int*>(a.meta + a.off_counts);
  int* starts = reinterpret_cast<int*>(a.meta + a.off_starts);
  int4* items = reinterpret_cast<int4*>(a.meta + a.off_items);

  // 1. per-batch lengths (and, for decode, the visible keys of its rows)
  long long vis = 0;
  for (int b = tid; b < B; b += kMetaThreads) {
    int q_off, s1, k_off, s2;
    if (a.layout_q == L_TND) {
      q_off = b ? a.cu_q[b - 1] : 0;
      s1 = a.cu_q[b] - q_off;
    } else {
      q_off = b * a.s1max;
      s1 = a.s1max;
    }
    if (a.layout_k == L_TND) {
      k_off = b ? a.cu_k[b - 1] : 0;
      s2 = a.cu_k[b] - k_off;
    } else if (a.layout_k == L_PA) {
      k_off = 0;
      s2 = a.seqused_k[b];
    } else {
      k_off = b * a.s2max;
      s2 = a.s2max;
    }
    bt[b] = int4{q_off, s1, k_off, s2};
    if (mode == kModeDecode)
      for (int i = 0; i < s1; ++i) vis += visible_limit(a.mask_mode, i, s1, s2);
  }
  // decode segment length from the total number of visible keys: one segment per
  // wave of a full GPU (kDecodeSegments, more if there are many rows); every row
  // adds at most one partial segment, so the count stays within the target.
  if (mode == kModeDecode) {
    long long rows = 0;
    for (int b = tid; b < B; b += kMetaThreads) rows += bt[b].y;
    for (int o = 32; o > 0; o >>= 1) {
      vis += __shfl_xor(vis, o);
      rows += __shfl_xor(rows, o);
    }
    if (lane == 0) {
      s_vis[wave] = vis;
      s_rows[wave] = rows;
    }
    __syncthreads();
    if (tid == 0) {
      long long tot = 0, nrows = 0;
      for (int w = 0; w < kMetaThreads / 64; ++w) {
        tot += s_vis[w];
        nrows += s_rows[w];
      }
      long long target = kDecodeSegments;
      while (target < 2 * nrows) target += kDecodeSegments;
      long long c = (tot + (target - nrows) - 1) / (target - nrows);
      c = (c + kTileKeys - 1) / kTileKeys * kTileKeys;
      s_chunk = (int)(c > a.chunk ? c : a.chunk);
    }
  } else if (tid == 0) {
    s_chunk = a.chunk;
  }
  __syncthreads();
  const int chunk = s_chunk;

  for (int b = tid; b < B; b += kMetaThreads) {
    const int4 rec = bt[b];
    int cnt = 0;
    if (mode == kModeDecode) {
      for (int i = 0; i < rec.y; ++i) cnt += cdiv(visible_limit(a.mask_mode, i, rec.y, rec.w), chunk);
    } else {
      cnt = cdiv(rec.y, a.rows_per_item);
    }
    counts[b] = cnt;
    if (B <= kRoundRobinMaxBatch) s_counts[b] = cnt;
  }
  __syncthreads();

  // 2. exclusive prefix of the counts (each thread scans a contiguous segment)
  const int seg = cdiv(B, kMetaThreads);
  const int b0 = tid * seg, b1 = min(b0 + seg, B);
  int local = 0;
  for (int b = b0; b < b1; ++b) local += counts[b];
  const int incl = wave_prefix_sum(local);
  if (lane == 63) s_part[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int w = 0; w < kMetaThreads / 64; ++w) {
      const int v = s_part[w];
      s_part[w] = acc;
      acc += v;
    }
    s_total = acc;
  }
  __syncthreads();
  int run = s_part[wave] + incl - local;
  for (int b = b0; b < b1; ++b) {
    starts[b] = run;
    run += counts[b];
  }
  const int total = min(s_total, a.max_items);
  if (tid == 0) {
    hdr->n_items = total;
    hdr->mode = mode;
    hdr->chunk = chunk;
    hdr->magic = kMetaMagic;
    hdr->batch = B;
    hdr->max_items = a.max_items;
  }
  __syncthreads();

  // 3. items
  for (int u = tid; u < total; u += kMetaThreads) {
    // batch of the u-th item in batch-major order: last b with starts[b] <= u
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (starts[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int r = u - starts[b];
    const int4 rec = bt[b];
    if (mode != kModeDecode) {
      const int cnt = counts[b];
      const int blk = cnt - 1 - r;                 // r = 0 is the last (costliest) block
      const int q0 = blk * a.rows_per_item;
      const int nrows = min(a.rows_per_item, rec.y - q0);
      int pos = u;
      if (B <= kRoundRobinMaxBatch) {
        // round-robin over batches, each batch walked from its last block:
        // pos = sum_b' min(r, cnt_b') + #{b' < b : cnt_b' > r}
        pos = 0;
        for (int bb = 0; bb < B; ++bb) {
          const int c = s_counts[bb];
          pos += min(r, c) + ((bb < b && c > r) ? 1 : 0);
        }
      }
      if (pos < a.max_items) items[pos] = int4{b, q0, nrows, 0};
    } else {
      int rest = r, i = 0, lim = 0;
      for (; i < rec.y; ++i) {
        lim = visible_limit(a.mask_mode, i, rec.y, rec.w);
        const int nch = cdiv(lim, chunk);
        if (rest < nch) break;
        rest -= nch;
      }
      const int k0 = rest * chunk;
      const int k1 = min(k0 + chunk, lim);
      items[u] = int4{b, i, k0, k1};
    }
  }
}

}  // namespace

hipError_t launch_metadata(const KArgs& a, int mode, hipStream_t s) {
  hipLaunchKernelGGL(metadata_kernel, dim3(1), dim3(kMetaThreads), 0, s, a, mode);
  return hipGetLastError();
}

}  // namespace li
