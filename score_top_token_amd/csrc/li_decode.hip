// Decode-shaped problems (at most a few query rows per batch, long key lists).
//
// A handful of query rows cannot fill 256 compute units row by row, so the keys
// of each row are cut into chunks (the work items of the metadata kernel).  The
// split kernel streams each chunk of K from HBM once, straight into MFMA B
// operands (no LDS round trip: every K byte is used by one row only), applies
// the ReLU / weight / head-sum epilogue, and stores each key's score as an
// order-preserving u32 into a dense per-row slot array in the workspace.  The
// select kernel then runs one workgroup per row: an exact 8-bit-digit radix
// select of the k-th largest key over the row (held in LDS when it fits), and
// a stable, block-wide compaction that writes the top-k in increasing key
// order, ties resolved toward smaller indices, and pads with -1 / -inf.
//
// The score follows the npu_lightning_indexer_pto page (formula under "功能说明")
// and the lightning_indexer page ("Function" steps 1-3, Constraints for the
// padding); paged keys are read through block_table (npu_lightning_indexer_pto
// page, block_table parameter).
#include "li_common_kernels.h"

namespace li {

namespace {

constexpr int kSplitWaves = 4;

template <int QK, int MB, int WT>
__global__ __launch_bounds__(256, 2) void split_kernel(KArgs a) {
  typedef Mma<QK> M;
  typedef typename M::frag F;
  const MetaHeader* hdr = reinterpret_cast<const MetaHeader*>(a.meta);
  if ((int)blockIdx.x >= hdr->n_items) return;
  const int4 item = reinterpret_cast<const int4*>(a.meta + a.off_items)[blockIdx.x];
  const int b = item.x, i = item.y, k0 = item.z, k1 = item.w;
  const int4 br = batch_rec(a, b);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t tok = (int64_t)br.x + i;

  F qf[MB][M::KSTEPS];
  float wv[MB][16];
  load_query<QK, MB, WT>(a, tok, lane, qf, wv);

  uint32_t* dst = a.ws + ((int64_t)b * a.s1max + i) * a.ws_row_stride;
  for (int base = k0 + wave * kTileKeys; base < k1; base += kSplitWaves * kTileKeys) {
    F kf[2][M::KSTEPS];
    int64_t slot[2] = {0, 0};
#pragma unroll
    for (int nb = 0; nb < 2; ++nb) {
      const int s = base + nb * 32 + (lane & 31);
      if (s < k1) {
        const unsigned char* row = key_row<QK>(a, b, br.z, s, &slot[nb]);
#pragma unroll
        for (int j = 0; j < M::KSTEPS; ++j) kf[nb][j] = load_frag_global<QK>(row + frag_off<QK>(lane, j));
      } else {
#pragma unroll
        for (int j = 0; j < M::KSTEPS; ++j) kf[nb][j] = zero_frag<QK>();
      }
    }
    f32x16 acc[MB][2];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      acc[mb][0] = f32x16{};
      acc[mb][1] = f32x16{};
    }
#pragma unroll
    for (int j = 0; j < M::KSTEPS; ++j)
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = M::mma(qf[mb][j], kf[nb][j], acc[mb][nb]);
    float tot = head_sum<MB>(acc, wv, lane);
    const int s = base + lane;
    if (s < k1) {
      if constexpr (QK == DT_FP8) {
        // both lane halves load every key of the tile, so lane l already holds the
        // slot of its own key (column l % 32 of block l / 32)
        tot *= a.k_descale[lane < 32 ? slot[0] : slot[1]];
      }
      dst[s] = f2key(tot);
    }
  }
}

// ---- block-wide helpers for the select kernel (1024 threads = 16 waves) ----

constexpr int kSelWaves = kSelectThreads / 64;

// exclusive prefix sum over the block; `tmp` holds kSelWaves ints of LDS
__device__ inline int block_exclusive_scan(int v, int* tmp, int* total) {
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int incl = wave_prefix_sum(v);
  if (l == 63) tmp[wave] = incl;
  __syncthreads();
  int wbase = 0, all = 0;
  for (int w = 0; w < kSelWaves; ++w) {
    const int t = tmp[w];
    if (w < wave) wbase += t;
    all += t;
  }
  __syncthreads();
  if (total) *total = all;
  return wbase + incl - v;
}

__global__ __launch_bounds__(kSelectThreads) void select_kernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int r = blockIdx.x;
  const int b = r / a.s1max, i = r - (r / a.s1max) * a.s1max;
  if (b >= a.batch) return;
  const int4 br = batch_rec(a, b);
  if (i >= br.y) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int lim = visible_limit(a.mask_mode, i, br.y, br.w);
  const int topk = a.topk;
  const int64_t tok = (int64_t)br.x + i;
  int32_t* oi = a.out_idx + tok * topk;
  float* ov = a.out_val ? a.out_val + tok * topk : nullptr;
  const uint32_t* src = a.ws + ((int64_t)b * a.s1max + i) * a.ws_row_stride;

  if (lim <= topk) {
    for (int e = tid; e < topk; e += kSelectThreads) {
      if (e < lim) {
        oi[e] = e;
        if (ov) ov[e] = key2f(src[e]);
      } else {
        oi[e] = -1;
        if (ov) ov[e] = -__builtin_inff();
      }
    }
    return;
  }

  uint32_t* whist = reinterpret_cast<uint32_t*>(smem);                // kSelWaves x 256
  int* scratch = reinterpret_cast<int*>(smem + kSelWaves * 256 * 4);   // 64 ints
  uint32_t* cache = reinterpret_cast<uint32_t*>(smem + kSelWaves * 256 * 4 + 256);
  const bool cached = lim <= kSelectCacheKeys;
  const uint32_t* keys = src;
  if (cached) {
    for (int e = tid; e < lim; e += kSelectThreads) cache[e] = src[e];
    keys = cache;
  }

  uint32_t prefix = 0, pmask = 0;
  int rem = topk;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int x = tid; x < kSelWaves * 256; x += kSelectThreads) whist[x] = 0;
    __syncthreads();
    uint32_t* mine = whist + wave * 256;
    for (int e = tid; e < lim; e += kSelectThreads) {
      const uint32_t u = keys[e];
      if ((u & pmask) == prefix) atomicAdd(&mine[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      uint32_t h[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        uint32_t t = 0;
        for (int w = 0; w < kSelWaves; ++w) t += whist[w * 256 + 4 * lane + q];
        h[q] = t;
      }
      const int s = (int)(h[0] + h[1] + h[2] + h[3]);
      const int suf = wave_suffix_sum(s);
      const int above = suf - s;
      if (above < rem && rem <= suf) {
        int acc = above, dgt = 4 * lane, gt = 0;
        bool done = false;
        for (int q = 3; q >= 0 && !done; --q) {
          if (acc + (int)h[q] >= rem) {
            dgt = 4 * lane + q;
            gt = acc;
            done = true;
          } else {
            acc += (int)h[q];
          }
        }
        scratch[0] = dgt;
        scratch[1] = gt;
      }
    }
    __syncthreads();
    const int dgt = scratch[0], gt = scratch[1];
    rem -= gt;
    prefix |= ((uint32_t)dgt) << shift;
    pmask |= 0xFFu << shift;
    __syncthreads();
  }
  const uint32_t kth = prefix;
  const int ties_needed = rem;

  // stable block-wide compaction: each thread owns a contiguous segment
  const int seg = (lim + kSelectThreads - 1) / kSelectThreads;
  const int e0 = tid * seg;
  const int e1 = e0 + seg < lim ? e0 + seg : lim;
  int ngt = 0, neq = 0;
  for (int e = e0; e < e1; ++e) {
    const uint32_t u = keys[e];
    ngt += u > kth;
    neq += u == kth;
  }
  const int eq_before = block_exclusive_scan(neq, scratch + 2, nullptr);
  int my_ties = ties_needed - eq_before;
  my_ties = my_ties < 0 ? 0 : (my_ties > neq ? neq : my_ties);
  const int pos0 = block_exclusive_scan(ngt + my_ties, scratch + 2 + kSelWaves, nullptr);
  int pos = pos0, tl = my_ties;
  for (int e = e0; e < e1; ++e) {
    const uint32_t u = keys[e];
    bool keep = u > kth;
    if (!keep && u == kth && tl > 0) {
      keep = true;
      --tl;
    }
    if (keep) {
      oi[pos] = e;
      if (ov) ov[pos] = key2f(u);
      ++pos;
    }
  }
  (void)lane;
}

template <int QK, int MB, int WT>
hipError_t launch_split(const KArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((split_kernel<QK, MB, WT>), dim3(grid), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <int QK, int MB>
hipError_t launch_split_w(const KArgs& a, int w_dtype, int grid, hipStream_t s) {
  return w_dtype == DT_FP32 ? launch_split<QK, MB, DT_FP32>(a, grid, s)
                            : launch_split<QK, MB, DT_BF16>(a, grid, s);
}

template <int QK>
hipError_t launch_split_mb(const KArgs& a, int w_dtype, int mblocks, int grid, hipStream_t s) {
  return mblocks == 1 ? launch_split_w<QK, 1>(a, w_dtype, grid, s)
                      : launch_split_w<QK, 2>(a, w_dtype, grid, s);
}

}  // namespace

hipError_t launch_decode(const KArgs& a, int qk_dtype, int w_dtype, int mblocks, int grid,
                         hipStream_t s) {
  switch (qk_dtype) {
    case DT_BF16: return launch_split_mb<DT_BF16>(a, w_dtype, mblocks, grid, s);
    case DT_FP16: return launch_split_mb<DT_FP16>(a, w_dtype, mblocks, grid, s);
    case DT_FP8: return launch_split_mb<DT_FP8>(a, w_dtype, mblocks, grid, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_select(const KArgs& a, int grid, size_t lds, hipStream_t s) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(select_kernel),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3(grid), dim3(kSelectThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace li
