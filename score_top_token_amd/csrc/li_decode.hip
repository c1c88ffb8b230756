// Decode-shaped problems (at most a few query rows per batch, long key lists).
//
// A handful of query rows cannot fill 256 compute units row by row, so the
// visible keys of all rows are cut into segments of about equal length (the
// work items of the metadata kernel).  The split kernel streams each segment of
// K from HBM once, straight into MFMA B operands (every K byte is used by one
// row only, so there is no LDS round trip), double-buffered in registers so the
// next tile's loads are in flight while the current tile is scored, applies the
// ReLU / weight / head-sum epilogue and stores each key's score into a dense
// per-row fp32 array in the workspace.  The select kernel then runs one
// workgroup per row: the exact bucket select of the k-th element (value
// descending, smaller key first on ties) over the row held in LDS, and a stable
// write of the top-k in ascending key order, padded with -1 / -inf.
//
// The score follows the npu_lightning_indexer_pto page (formula under "功能说明")
// and the lightning_indexer page ("Function" steps 1-3, Constraints for the
// padding); paged keys are read through block_table (npu_lightning_indexer_pto
// page, block_table parameter).
#include "li_common_kernels.h"
#include "li_select.h"

namespace li {

namespace {

template <int QK, bool PAGED>
__device__ inline void load_key_frags(const KArgs& a, int b, int k_off, int base, int k1, int lane,
                                      typename Mma<QK>::frag (&kf)[2][Mma<QK>::KSTEPS],
                                      int64_t& slot) {
  typedef Mma<QK> M;
  slot = 0;
#pragma unroll
  for (int nb = 0; nb < 2; ++nb) {
    const int s = base + nb * 32 + (lane & 31);
    if (s < k1) {
      const unsigned char* row = key_row<QK, PAGED>(a, b, k_off, s);
#pragma unroll
      for (int j = 0; j < M::KSTEPS; ++j) kf[nb][j] = load_frag_global<QK>(row + frag_off<QK>(lane, j));
      // lane l reports key base + l: column l % 32 of block l / 32
      if constexpr (QK == DT_FP8) {
        if (nb == (lane >> 5)) slot = key_slot<PAGED>(a, b, k_off, s);
      }
    } else {
#pragma unroll
      for (int j = 0; j < M::KSTEPS; ++j) kf[nb][j] = zero_frag<QK>();
    }
  }
}

template <int QK, int MB>
__device__ inline float score_tile_regs(const typename Mma<QK>::frag (&qf)[MB][Mma<QK>::KSTEPS],
                                        const typename Mma<QK>::frag (&kf)[2][Mma<QK>::KSTEPS],
                                        const float (&wv)[MB][16], int lane) {
  typedef Mma<QK> M;
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
  return head_sum<MB>(acc, wv, lane);
}

// One wave per segment (item): waves of a workgroup work independently.
template <int QK, int MB, int WT, bool PAGED>
__global__ __launch_bounds__(kDecodeWaves * 64, 1) void split_kernel(KArgs a) {
  typedef Mma<QK> M;
  typedef typename M::frag F;
  constexpr int STEP = kTileKeys;
  const MetaHeader* hdr = reinterpret_cast<const MetaHeader*>(a.meta);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int it = blockIdx.x * kDecodeWaves + wave;
  if (it >= hdr->n_items) return;
  const int4 item = reinterpret_cast<const int4*>(a.meta + a.off_items)[it];
  const int b = item.x, i = item.y, k0 = item.z, k1 = item.w;
  const int4 br = batch_rec(a, b);
  const int64_t tok = (int64_t)br.x + i;

  F qf[MB][M::KSTEPS];
  float wv[MB][16];
  load_query<QK, MB, WT>(a, tok, lane, qf, wv);
  float* dst = a.ws + ((int64_t)b * a.s1max + i) * a.ws_row_stride;

  auto finish = [&](int base, float tot, int64_t slot) {
    const int s = base + lane;
    if (s < k1) {
      if constexpr (QK == DT_FP8) tot *= a.k_descale[slot];
      // -0 -> +0; NaN (only from NaN inputs) -> -inf keeps the scores ordered
      dst[s] = tot == 0.0f ? 0.0f : (tot != tot ? -__builtin_inff() : tot);
    }
  };

  F ka[2][M::KSTEPS], kb[2][M::KSTEPS];
  int64_t sa = 0, sb = 0;
  int base = k0;
  if (base < k1) load_key_frags<QK, PAGED>(a, b, br.z, base, k1, lane, ka, sa);
  while (base < k1) {
    if (base + STEP < k1) load_key_frags<QK, PAGED>(a, b, br.z, base + STEP, k1, lane, kb, sb);
    finish(base, score_tile_regs<QK, MB>(qf, ka, wv, lane), sa);
    base += STEP;
    if (base >= k1) break;
    if (base + STEP < k1) load_key_frags<QK, PAGED>(a, b, br.z, base + STEP, k1, lane, ka, sa);
    finish(base, score_tile_regs<QK, MB>(qf, kb, wv, lane), sb);
    base += STEP;
  }
}

// ---------------------------------------------------------------------------
// block-wide helpers of the select kernel (1024 threads = 16 waves)
// ---------------------------------------------------------------------------
constexpr int kSelWaves = kSelectThreads / 64;
constexpr int kNB = kSelectBuckets;

struct SelShared {
  int misc[64];           // 0: bucket, 1: above, 2: count, 3: gathered, 4..5: fb/eb, 8..: scan
  float cand_f[kSelSmall];
  uint32_t cand_e[kSelSmall];
  uint32_t hist[kNB];
};

__device__ inline float block_min_f(float v, int* tmp) {
  v = wave_min_f(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) tmp[w] = __float_as_int(v);
  __syncthreads();
  float r = __int_as_float(tmp[0]);
  for (int x = 1; x < kSelWaves; ++x) r = fminf(r, __int_as_float(tmp[x]));
  __syncthreads();
  return r;
}
__device__ inline float block_max_f(float v, int* tmp) {
  v = wave_max_f(v);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) tmp[w] = __float_as_int(v);
  __syncthreads();
  float r = __int_as_float(tmp[0]);
  for (int x = 1; x < kSelWaves; ++x) r = fmaxf(r, __int_as_float(tmp[x]));
  __syncthreads();
  return r;
}
__device__ inline uint32_t block_min_u(uint32_t v, int* tmp) {
  v = wave_min_u(v);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = (int)v;
  __syncthreads();
  uint32_t r = (uint32_t)tmp[0];
  for (int x = 1; x < kSelWaves; ++x) r = min(r, (uint32_t)tmp[x]);
  __syncthreads();
  return r;
}
__device__ inline uint32_t block_max_u(uint32_t v, int* tmp) {
  v = wave_max_u(v);
  if ((threadIdx.x & 63) == 0) tmp[threadIdx.x >> 6] = (int)v;
  __syncthreads();
  uint32_t r = (uint32_t)tmp[0];
  for (int x = 1; x < kSelWaves; ++x) r = max(r, (uint32_t)tmp[x]);
  __syncthreads();
  return r;
}

// exclusive prefix over the 16 waves of a per-wave (uniform) value
__device__ inline int block_wave_prefix(int v, int* tmp, int* total) {
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) tmp[w] = v;
  __syncthreads();
  int before = 0, all = 0;
  for (int x = 0; x < kSelWaves; ++x) {
    const int t = tmp[x];
    before += x < w ? t : 0;
    all += t;
  }
  __syncthreads();
  if (total) *total = all;
  return before;
}

// Bucket of the element of rank r from the top of hist[0, kNB): thread t owns
// buckets 2t, 2t+1.  Writes bucket / above / count to sh.misc[0..2].
__device__ inline void block_find_bucket(SelShared& sh, int r) {
  const int t = threadIdx.x, w = t >> 6;
  const uint32_t h0 = sh.hist[2 * t], h1 = sh.hist[2 * t + 1];
  const int s = (int)(h0 + h1);
  const int wsuf = wave_suffix_sum(s);                 // within the wave
  if ((t & 63) == 0) sh.misc[8 + w] = wsuf;            // wave total (lane 0 holds the full sum)
  __syncthreads();
  int higher = 0;
  for (int x = w + 1; x < kSelWaves; ++x) higher += sh.misc[8 + x];
  const int suf = wsuf + higher;
  const int ab = suf - s;
  if (ab < r && r <= suf) {
    if (ab + (int)h1 >= r) {
      sh.misc[0] = 2 * t + 1;
      sh.misc[1] = ab;
      sh.misc[2] = (int)h1;
    } else {
      sh.misc[0] = 2 * t;
      sh.misc[1] = ab + (int)h1;
      sh.misc[2] = (int)h0;
    }
  }
  __syncthreads();
}

struct FBucketN {
  float lo2, scale;
  __device__ FBucketN(float lo, float hi) {
    lo2 = lo * 0.5f;
    scale = fminf((float)kNB / (hi * 0.5f - lo2), 3.0e38f);
  }
  __device__ uint32_t operator()(float f) const {
    const float x = fminf((f * 0.5f - lo2) * scale, (float)(kNB - 1));
    return (uint32_t)fmaxf(x, 0.0f);
  }
};

struct UBucketN {
  uint32_t ulo;
  int shift;
  __device__ UBucketN(uint32_t lo, uint32_t hi) : ulo(lo) {
    const uint32_t span = hi - lo;
    const int bits = span ? 32 - __clz(span) : 0;
    shift = bits > 11 ? bits - 11 : 0;
  }
  __device__ uint32_t operator()(uint32_t u) const {
    const uint32_t b = (u - ulo) >> shift;
    return b > (uint32_t)(kNB - 1) ? (uint32_t)(kNB - 1) : b;
  }
};

// gathers the (<= kSelSmall) candidates with in(f) into sh.cand_*, then wave 0
// ranks them; the k-th element lands in sh.misc[4..5]
template <class Pred>
__device__ inline void block_gather_rank(SelShared& sh, const float* vals, int n, int r, Pred in) {
  if (threadIdx.x == 0) sh.misc[3] = 0;
  __syncthreads();
  for (int e = threadIdx.x; e < n; e += kSelectThreads) {
    const float f = vals[e];
    if (in(f)) {
      const int slot = atomicAdd(&sh.misc[3], 1);
      if (slot < kSelSmall) {
        sh.cand_f[slot] = f;
        sh.cand_e[slot] = (uint32_t)e;
      }
    }
  }
  __syncthreads();
  if (threadIdx.x < 64) {
    const int m = min(sh.misc[3], kSelSmall);
    const int l = threadIdx.x;
    const float cf = l < m ? sh.cand_f[l] : 0.0f;
    const uint32_t ce = l < m ? sh.cand_e[l] : 0u;
    float fb;
    uint32_t eb;
    wave_rank_small(cf, ce, m, r, fb, eb);
    if (l == 0) {
      sh.misc[4] = __float_as_int(fb);
      sh.misc[5] = (int)eb;
    }
  }
  __syncthreads();
}

// the r-th entry (index order) whose key equals u; writes fb / eb into sh.misc[4..5]
__device__ inline void block_rth_equal(SelShared& sh, const float* vals, int n, int r, uint32_t u) {
  const int w = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int seg = ((n + kSelWaves - 1) / kSelWaves + 63) / 64 * 64;
  const int e0 = w * seg, e1 = min(n, e0 + seg);
  int cnt = 0;
  for (int p0 = e0; p0 < e1; p0 += 64) {
    const int p = p0 + l;
    cnt += __popcll(ballot(p < e1 && f2key(vals[p]) == u));
  }
  const int before = block_wave_prefix(cnt, sh.misc + 8, nullptr);
  if (before < r && r <= before + cnt) {
    int seen = before;
    for (int p0 = e0; p0 < e1; p0 += 64) {
      const int p = p0 + l;
      const bool eq = p < e1 && f2key(vals[p]) == u;
      const uint64_t m = ballot(eq);
      if (seen + __popcll(m) >= r) {
        if (eq && seen + mbcnt(m) == r - 1) {
          sh.misc[4] = (int)u;
          sh.misc[5] = p;
        }
        break;
      }
      seen += __popcll(m);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) sh.misc[4] = __float_as_int(key2f(u));
  __syncthreads();
}

// k-th element of vals[0, n) in (value desc, index asc) order -> sh.misc[4..5]
__device__ void block_kth(SelShared& sh, const float* vals, int n, int k, float lo, float hi) {
  int r = k;
  uint32_t ulo, uhi;
  if (lo < hi) {
    const FBucketN fbk(lo, hi);
    for (int x = threadIdx.x; x < kNB; x += kSelectThreads) sh.hist[x] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += kSelectThreads) atomicAdd(&sh.hist[fbk(vals[e])], 1u);
    __syncthreads();
    block_find_bucket(sh, r);
    const uint32_t B = (uint32_t)sh.misc[0];
    const int above = sh.misc[1], cnt = sh.misc[2];
    r -= above;
    __syncthreads();
    if (cnt <= kSelSmall) {
      block_gather_rank(sh, vals, n, r, [&](float f) { return fbk(f) == B; });
      return;
    }
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int e = threadIdx.x; e < n; e += kSelectThreads) {
      const float f = vals[e];
      if (fbk(f) == B) {
        const uint32_t u = f2key(f);
        mn = min(mn, u);
        mx = max(mx, u);
      }
    }
    ulo = block_min_u(mn, sh.misc + 8);
    uhi = block_max_u(mx, sh.misc + 8);
  } else {
    ulo = uhi = f2key(lo);
  }
  for (;;) {
    if (ulo == uhi) {
      block_rth_equal(sh, vals, n, r, ulo);
      return;
    }
    const UBucketN ubk(ulo, uhi);
    for (int x = threadIdx.x; x < kNB; x += kSelectThreads) sh.hist[x] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += kSelectThreads) {
      const uint32_t u = f2key(vals[e]);
      if (u >= ulo && u <= uhi) atomicAdd(&sh.hist[ubk(u)], 1u);
    }
    __syncthreads();
    block_find_bucket(sh, r);
    const int B = sh.misc[0], above = sh.misc[1], cnt = sh.misc[2];
    r -= above;
    __syncthreads();
    const uint32_t nlo = ulo + ((uint32_t)B << ubk.shift);
    uint32_t nhi = (B == kNB - 1) ? uhi : nlo + ((1u << ubk.shift) - 1u);
    if (nhi > uhi) nhi = uhi;
    if (cnt <= kSelSmall && nlo != nhi) {
      block_gather_rank(sh, vals, n, r, [&](float f) {
        const uint32_t u = f2key(f);
        return u >= nlo && u <= nhi;
      });
      return;
    }
    ulo = nlo;
    uhi = nhi;
  }
}

__global__ __launch_bounds__(kSelectThreads) void select_kernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SelShared& sh = *reinterpret_cast<SelShared*>(smem);
  float* cache = reinterpret_cast<float*>(smem + sizeof(SelShared));
  const int r = blockIdx.x;
  const int b = r / a.s1max, i = r - (r / a.s1max) * a.s1max;
  if (b >= a.batch) return;
  const int4 br = batch_rec(a, b);
  if (i >= br.y) return;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
  const int lim = visible_limit(a.mask_mode, i, br.y, br.w);
  const int topk = a.topk;
  const int64_t tok = (int64_t)br.x + i;
  int32_t* oi = a.out_idx + tok * topk;
  float* ov = a.out_val ? a.out_val + tok * topk : nullptr;
  const float* src = a.ws + ((int64_t)b * a.s1max + i) * a.ws_row_stride;

  if (lim <= topk) {
    for (int e = tid; e < topk; e += kSelectThreads) {
      if (e < lim) {
        oi[e] = e;
        if (ov) ov[e] = src[e];
      } else {
        oi[e] = -1;
        if (ov) ov[e] = -__builtin_inff();
      }
    }
    return;
  }
  const bool cached = lim <= kSelectCacheKeys;
  float mn = __builtin_inff(), mx = -__builtin_inff();
  for (int e = tid; e < lim; e += kSelectThreads) {
    const float f = src[e];
    if (cached) cache[e] = f;
    mn = fminf(mn, f);
    mx = fmaxf(mx, f);
  }
  const float lo = block_min_f(mn, sh.misc + 8);
  const float hi = block_max_f(mx, sh.misc + 8);
  const float* vals = cached ? cache : src;
  block_kth(sh, vals, lim, topk, lo, hi);
  const float fb = __int_as_float(sh.misc[4]);
  const uint32_t eb = (uint32_t)sh.misc[5];
  __syncthreads();

  // stable write: each wave owns a contiguous, 64-aligned segment of the row
  const int seg = ((lim + kSelWaves - 1) / kSelWaves + 63) / 64 * 64;
  const int e0 = w * seg, e1 = min(lim, e0 + seg);
  int kept = 0;
  for (int p0 = e0; p0 < e1; p0 += 64) {
    const int p = p0 + l;
    bool keep = false;
    if (p < e1) {
      const float f = vals[p];
      keep = f > fb || (f == fb && (uint32_t)p <= eb);
    }
    kept += __popcll(ballot(keep));
  }
  int pos = block_wave_prefix(kept, sh.misc + 8, nullptr);
  for (int p0 = e0; p0 < e1; p0 += 64) {
    const int p = p0 + l;
    float f = 0.0f;
    bool keep = false;
    if (p < e1) {
      f = vals[p];
      keep = f > fb || (f == fb && (uint32_t)p <= eb);
    }
    const uint64_t m = ballot(keep);
    if (keep) {
      const int o = pos + mbcnt(m);
      if (o < topk) {                      // bounded whatever the data
        oi[o] = p;
        if (ov) ov[o] = f;
      }
    }
    pos += __popcll(m);
  }
}

template <int QK, int MB, int WT, bool PAGED>
hipError_t launch_split(const KArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((split_kernel<QK, MB, WT, PAGED>), dim3(grid), dim3(kDecodeWaves * 64), 0, s, a);
  return hipGetLastError();
}

template <int QK, int MB, int WT>
hipError_t launch_split_p(const KArgs& a, bool paged, int grid, hipStream_t s) {
  return paged ? launch_split<QK, MB, WT, true>(a, grid, s)
               : launch_split<QK, MB, WT, false>(a, grid, s);
}

template <int QK, int MB>
hipError_t launch_split_w(const KArgs& a, int w_dtype, bool paged, int grid, hipStream_t s) {
  return w_dtype == DT_FP32 ? launch_split_p<QK, MB, DT_FP32>(a, paged, grid, s)
                            : launch_split_p<QK, MB, DT_BF16>(a, paged, grid, s);
}

template <int QK>
hipError_t launch_split_mb(const KArgs& a, int w_dtype, int mblocks, bool paged, int grid,
                           hipStream_t s) {
  return mblocks == 1 ? launch_split_w<QK, 1>(a, w_dtype, paged, grid, s)
                      : launch_split_w<QK, 2>(a, w_dtype, paged, grid, s);
}

}  // namespace

size_t select_shared_bytes() { return sizeof(SelShared); }

hipError_t launch_decode(const KArgs& a, int qk_dtype, int w_dtype, int mblocks, bool paged,
                         int grid, hipStream_t s) {
  switch (qk_dtype) {
    case DT_BF16: return launch_split_mb<DT_BF16>(a, w_dtype, mblocks, paged, grid, s);
    case DT_FP16: return launch_split_mb<DT_FP16>(a, w_dtype, mblocks, paged, grid, s);
    case DT_FP8: return launch_split_mb<DT_FP8>(a, w_dtype, mblocks, paged, grid, s);
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
