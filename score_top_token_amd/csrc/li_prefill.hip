// Prefill kernel: scores of a block of up to 4 query rows against every
// visible key, fused with an exact streaming top-k per row.
//
// Score (npu_lightning_indexer_pto page, formula under "功能说明"; lightning_indexer
// page, "Function" steps 1-3): I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:]).
// The Q.K^T tile is an MFMA contraction with heads on M and keys on N; ReLU, the
// weights and the head sum run on the fp32 accumulators in registers.
//
// Top-k (same pages, step 3; padding rule from the Constraints section): each
// wave owns one query row and a candidate list of `cap` (key, index) slots in
// LDS.  Scores arrive in increasing key order and are appended in that order
// when they beat the running threshold; when the list is full an exact wave
// radix select finds the k-th largest key, a stable compaction keeps exactly k
// entries (ties resolved toward smaller key indices) and the threshold rises to
// that k-th key.  The list therefore stays sorted by key index, which makes the
// index tie-break a plain prefix count.  The full score matrix never leaves the
// chip.
#include "li_common_kernels.h"

namespace li {

namespace {

constexpr int kWaves = kRowsPerItem;

// Keeps exactly k of the n candidates (the top k, ties to smaller indices),
// preserving order.  Writes to dst (LDS list or output row) at positions
// 0..k-1; values go to dval when non-null.  Returns the k-th key.
template <bool TO_GLOBAL>
__device__ uint32_t select_keep(uint32_t* keysU, uint32_t* keysI, int n, int k, uint32_t* hist,
                                int32_t* gidx, float* gval) {
  const int l = lane_id();
  uint32_t kth;
  int ties;
  wave_radix_select(keysU, n, k, hist, kth, ties);
  int kept = 0;
  for (int e0 = 0; e0 < n; e0 += 64) {
    const int e = e0 + l;
    uint32_t u = 0, ix = 0;
    if (e < n) {
      u = keysU[e];
      ix = keysI[e];
    }
    const bool gt = e < n && u > kth;
    const bool eq = e < n && u == kth;
    const uint64_t em = ballot(eq);
    const bool keep = gt || (eq && mbcnt(em) < ties);
    const int ecnt = __popcll(em);
    ties -= ecnt < ties ? ecnt : ties;
    const uint64_t km = ballot(keep);
    wave_sync();
    if (keep) {
      const int pos = kept + mbcnt(km);
      if constexpr (TO_GLOBAL) {
        gidx[pos] = (int32_t)ix;
        if (gval) gval[pos] = key2f(u);
      } else {
        keysU[pos] = u;
        keysI[pos] = ix;
      }
    }
    kept += __popcll(km);
    wave_sync();
  }
  return kth;
}

template <int QK, int MB, int WT>
__global__ __launch_bounds__(256, 1) void prefill_kernel(KArgs a) {
  typedef Mma<QK> M;
  typedef typename M::frag F;
  constexpr int TILE_BYTES = kTileKeys * M::RB;
  constexpr int NCH = M::RB / 16;                  // 16-byte chunks per key row
  constexpr int LOADS = kTileKeys * NCH / 256;     // chunks per thread per tile

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  const MetaHeader* hdr = reinterpret_cast<const MetaHeader*>(a.meta);
  if ((int)blockIdx.x >= hdr->n_items) return;
  const int4 item = reinterpret_cast<const int4*>(a.meta + a.off_items)[blockIdx.x];
  const int b = item.x, q0 = item.y, nrows = item.z;
  const int4 br = batch_rec(a, b);                 // q_off, s1, k_off, s2
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cap = a.cap, topk = a.topk;

  unsigned char* ktile = smem;
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + 2 * TILE_BYTES) + wave * 256;
  uint32_t* listU = reinterpret_cast<uint32_t*>(smem + 2 * TILE_BYTES + kWaves * 256 * 4) + wave * cap;
  uint32_t* listI = listU + kWaves * cap;

  const bool has_row = wave < nrows;
  const int i = q0 + wave;
  const int lim = has_row ? visible_limit(a.mask_mode, i, br.y, br.w) : 0;
  // the visible limit never decreases with the row, so the last row bounds the block
  const int kend = visible_limit(a.mask_mode, q0 + nrows - 1, br.y, br.w);
  const int ntiles = (kend + kTileKeys - 1) / kTileKeys;
  const int64_t tok = (int64_t)br.x + i;

  F qf[MB][M::KSTEPS];
  float wv[MB][16];
  if (has_row) {
    load_query<QK, MB, WT>(a, tok, lane, qf, wv);
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int j = 0; j < M::KSTEPS; ++j) qf[mb][j] = zero_frag<QK>();
#pragma unroll
      for (int r = 0; r < 16; ++r) wv[mb][r] = 0.0f;
    }
  }

  i32x4 pre[LOADS];
  auto gload = [&](int t) {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int id = tid + 256 * r;
      const int key = id / NCH, c = id % NCH;
      const int s = t * kTileKeys + key;
      if (s < kend) {
        const unsigned char* row = key_row<QK>(a, b, br.z, s, nullptr);
        pre[r] = *reinterpret_cast<const i32x4*>(row + c * 16);
      } else {
        pre[r] = i32x4{0, 0, 0, 0};
      }
    }
  };
  auto lstore = [&](int buf) {
    unsigned char* dst = ktile + buf * TILE_BYTES;
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int id = tid + 256 * r;
      const int key = id / NCH, c = id % NCH;
      *reinterpret_cast<i32x4*>(dst + lds_chunk_off<QK>(key, c)) = pre[r];
    }
  };

  int count = 0;          // candidates in this wave's list (wave-uniform)
  uint32_t thr = 0;       // a new key must exceed this to enter (0: accept all)

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    if (t + 1 < ntiles) gload(t + 1);
    const int base = t * kTileKeys;
    if (base < lim) {
      const unsigned char* tile = ktile + (t & 1) * TILE_BYTES;
      f32x16 acc[MB][2];
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        acc[mb][0] = f32x16{};
        acc[mb][1] = f32x16{};
      }
#pragma unroll
      for (int j = 0; j < M::KSTEPS; ++j) {
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          const F kb = load_frag_lds<QK>(tile, nb * 32 + (lane & 31), lane, j);
#pragma unroll
          for (int mb = 0; mb < MB; ++mb) acc[mb][nb] = M::mma(qf[mb][j], kb, acc[mb][nb]);
        }
      }
      float tot = head_sum<MB>(acc, wv, lane);
      const int s = base + lane;
      const bool valid = s < lim;
      if constexpr (QK == DT_FP8) {
        int64_t slot = 0;
        if (valid) {
          key_row<QK>(a, b, br.z, s, &slot);
          tot *= a.k_descale[slot];
        }
      }
      const uint32_t u = f2key(tot);
      bool want = valid && u > thr;
      uint64_t m = ballot(want);
      int c = __popcll(m);
      if (c > 0) {
        if (count + c > cap) {
          thr = select_keep<false>(listU, listI, count, topk, hist, nullptr, nullptr);
          count = topk;
          want = valid && u > thr;
          m = ballot(want);
          c = __popcll(m);
        }
        if (want) {
          const int pos = count + mbcnt(m);
          listU[pos] = u;
          listI[pos] = (uint32_t)s;
        }
        count += c;
      }
      wave_sync();
    }
    if (t + 1 < ntiles) lstore((t + 1) & 1);
    __syncthreads();
  }

  if (!has_row) return;
  int32_t* oi = a.out_idx + tok * topk;
  float* ov = a.out_val ? a.out_val + tok * topk : nullptr;
  int n = count;
  if (count > topk) {
    select_keep<true>(listU, listI, count, topk, hist, oi, ov);
    n = topk;
  } else {
    for (int e = lane; e < count; e += 64) {
      oi[e] = (int32_t)listI[e];
      if (ov) ov[e] = key2f(listU[e]);
    }
  }
  for (int e = n + lane; e < topk; e += 64) {
    oi[e] = -1;
    if (ov) ov[e] = -__builtin_inff();
  }
}

template <int QK, int MB, int WT>
hipError_t launch_one(const KArgs& a, int grid, size_t lds, hipStream_t s) {
  auto fn = prefill_kernel<QK, MB, WT>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(256), lds, s, a);
  return hipGetLastError();
}

template <int QK, int MB>
hipError_t launch_w(const KArgs& a, int w_dtype, int grid, size_t lds, hipStream_t s) {
  return w_dtype == DT_FP32 ? launch_one<QK, MB, DT_FP32>(a, grid, lds, s)
                            : launch_one<QK, MB, DT_BF16>(a, grid, lds, s);
}

template <int QK>
hipError_t launch_mb(const KArgs& a, int w_dtype, int mblocks, int grid, size_t lds,
                     hipStream_t s) {
  return mblocks == 1 ? launch_w<QK, 1>(a, w_dtype, grid, lds, s)
                      : launch_w<QK, 2>(a, w_dtype, grid, lds, s);
}

}  // namespace

hipError_t launch_prefill(const KArgs& a, int qk_dtype, int w_dtype, int mblocks, int grid,
                          size_t lds, hipStream_t s) {
  switch (qk_dtype) {
    case DT_BF16: return launch_mb<DT_BF16>(a, w_dtype, mblocks, grid, lds, s);
    case DT_FP16: return launch_mb<DT_FP16>(a, w_dtype, mblocks, grid, lds, s);
    case DT_FP8: return launch_mb<DT_FP8>(a, w_dtype, mblocks, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace li
