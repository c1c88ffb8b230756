// Decode-shaped problems (at most a few query rows per batch, long key lists).
//
// A handful of query rows cannot fill 256 compute units row by row, so the
// visible keys of all rows are cut into segments of about equal length (the
// work items of the metadata kernel).  The split kernel streams each segment of
// K from HBM once with coalesced loads, several tiles ahead of the compute,
// turns each tile into MFMA B operands through a per-wave LDS buffer, applies
// the ReLU / weight / head-sum epilogue and stores each key's score into a
// dense per-row fp32 array in the workspace.  The select kernel then runs one
// workgroup per row: the exact bucket select of the k-th element (value
// descending, smaller key first on ties) over the row held in registers, and a stable
// write of the top-k in ascending key order, padded with -1 / -inf.
//
// The score follows the npu_lightning_indexer_pto page (formula under "功能说明")
// and the lightning_indexer page ("Function" steps 1-3, Constraints for the
// padding); paged keys are read through block_table (npu_lightning_indexer_pto
// page, block_table parameter).
#include "li_pipe.h"
#include "li_select.h"

namespace li {

namespace {

constexpr int kDecodeDepth = 4;   // 32-key tiles in flight per wave (even)

// One wave per segment (item); the waves of a workgroup work independently.
// The segment's K streams through a ring of kDecodeDepth register sets filled
// by coalesced 16-byte loads (a 1 KiB run of K per instruction), so about
// kDecodeDepth * 32 keys are in flight per wave.  Each tile passes through the
// wave's own LDS buffer to reach the MFMA operand layout; its MFMAs are
// interleaved with the epilogue of the previous tile.
// One wave per SIMD by design (a 4-deep register ring of 32-key tiles): the
// attribute keeps the compiler from trading that ring for occupancy.
template <int QK, int MB, int WT, int KL>
__global__ __launch_bounds__(kDecodeWaves * 64, 1) __attribute__((amdgpu_waves_per_eu(1, 1)))
void split_kernel(KArgs a) {
  typedef Mma<QK> M;
  typedef typename M::frag F;
  constexpr int D = kDecodeDepth;
  constexpr int TILE = kPipeKeys * M::RB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if (!check_meta(a)) return;
  const MetaHeader* hdr = reinterpret_cast<const MetaHeader*>(a.meta);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int it = blockIdx.x * kDecodeWaves + wave;
  if (it >= hdr->n_items) return;
  const int4 item = reinterpret_cast<const int4*>(a.meta + a.off_items)[it];
  const int b = item.x, i = item.y, k0 = item.z, k1 = item.w;
  if (k0 >= k1) return;                    // an empty item (padding of the work list)
  const int4 br = batch_rec(a, b);
  const int64_t tok = (int64_t)br.x + i;
  unsigned char* tile = smem + wave * TILE;
  static_assert(q_stage_bytes<QK>() <= TILE, "a 32-head query block fits the wave's tile");

  PipeStage<QK, KL, 64, D> st;
  st.prefetch_table(a, b, k0);
  F qf[MB][M::KSTEPS];
  float wv[MB][16];
  // the query goes through the wave's LDS tile (coalesced loads), with the K
  // ring's first loads issued behind its loads
  auto fill_ring = [&]() __attribute__((always_inline)) {
    static_for<D>([&](auto set) {
      constexpr int S = decltype(set)::value;
      st.template load<S>(a, b, br.z, k0 + S * kPipeKeys, k1, lane);
    });
  };
  load_query<QK, MB, WT, true>(a, tok, lane, qf, wv, tile, fill_ring);
  float* dst = a.ws + ((int64_t)b * a.s1max + i) * a.ws_row_stride;

  // score of tile t: lanes 0-31 carry keys k0 + 32 t + lane.  The segment's
  // minimum and maximum stored score go to seg_mm, so that the select kernel
  // knows each row's range before it reads the row.
  float vmin = __builtin_inff(), vmax = -__builtin_inff();
  auto emit = [&](int t, float tot, float ds) {
    const int s = k0 + t * kPipeKeys + lane;
    if (lane < 32 && s < k1) {
      if constexpr (QK == DT_FP8) tot *= ds;
      // -0 -> +0; NaN (only from NaN inputs) -> -inf keeps the scores ordered
      const float v = tot == 0.0f ? 0.0f : (tot != tot ? -__builtin_inff() : tot);
      dst[s] = v;
      vmin = fminf(vmin, v);
      vmax = fmaxf(vmax, v);
    }
  };

  const int ntiles = (k1 - k0 + kPipeKeys - 1) / kPipeKeys;
  f32x16 accA[MB], accB[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accA[mb] = f32x16{};
    accB[mb] = f32x16{};
  }
  float dprev = 1.0f;

  // Step t (ring set S = t % D): tile t from set S into LDS, refill set S with
  // tile t + D, MFMAs of tile t into one accumulator set interleaved with the
  // epilogue of tile t - 1 from the other.
  auto step = [&](auto set, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(set)::value;
    f32x16(&cur)[MB] = (S & 1) ? accB : accA;
    f32x16(&prev)[MB] = (S & 1) ? accA : accB;
    st.template store<S>(tile, lane);
    const float dcur = st.dsc[S];
    st.template load<S>(a, b, br.z, k0 + (t + D) * kPipeKeys, k1, lane);
    wave_sync();
    F kb[M::KSTEPS];
    read_tile_frags<QK>(tile, lane, kb);
    mma_tile<QK, MB>(qf, kb, cur);
    const float prev_score = block_score<MB, QK != DT_FP8>(prev, wv);
    pipe_schedule<QK, MB>();
    if (t > 0) emit(t - 1, prev_score, dprev);
    dprev = dcur;
    wave_sync();
  };
  // Full groups of D steps run unconditionally, so every step issues the same
  // loads and the ring never drains; the last tiles follow one by one.
  int t = 0;
  for (; t + D <= ntiles; t += D) static_for<D>([&](auto set) { step(set, t + decltype(set)::value); });
  static_for<D - 1>([&](auto set) {
    if (t + decltype(set)::value < ntiles) step(set, t + decltype(set)::value);
  });
  const int last = ntiles - 1;
  constexpr bool kSwap = QK != DT_FP8;
  emit(last, (last & 1) ? block_score<MB, kSwap>(accB, wv) : block_score<MB, kSwap>(accA, wv), dprev);
  vmin = wave_min_f(vmin);
  vmax = wave_max_f(vmax);
  if (lane == 0) {
    float* mm = a.seg_mm + ((int64_t)b * a.s1max + i) * a.seg_mm_stride * 2 + 2 * (k0 / hdr->chunk);
    mm[0] = vmin;
    mm[1] = vmax;
  }
}

// ---------------------------------------------------------------------------
// block-wide helpers of the select kernel (1024 threads = 16 waves)
// ---------------------------------------------------------------------------
constexpr int kSelWaves = kSelectThreads / 64;
constexpr int kNB = kSelectBuckets;
constexpr int kKeptSlot = 24;   // sh.misc[kKeptSlot + w]: kept elements of wave w's segment

struct SelShared {
  int misc[64];           // 0: bucket, 1: above, 2: count, 3: gathered, 4..5: fb/eb,
                          // 6: kept counts ready, 8..23: scan, 24..39: kept per wave
  float cand_f[kSelSmall];
  uint32_t cand_e[kSelSmall];
  uint32_t hist[kNB + 64];   // + one discard bin per lane, so skipped elements never collide
};

// histogram slot of an element: its bucket, or the lane's discard bin
__device__ inline uint32_t hist_slot(bool in, uint32_t bucket) {
  return in ? bucket : (uint32_t)kNB + (threadIdx.x & 63);
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

// ---------------------------------------------------------------------------
// Row views.  The select reaches the scores of a row through two traversals:
//   each(f)    : f(e, valid, v) covering every element e of the row once (with
//                valid set) in any order, plus padding calls with valid false;
//   ordered(f) : wave w walks its contiguous segment of the row in index order,
//                64 elements per step, calling f(p, valid, v) with lane l
//                holding element p = step start + l.
// The segment of wave w is [w * seg, min(n, (w + 1) * seg)), seg a multiple of
// 64 of about n / 16.
// ---------------------------------------------------------------------------
__device__ inline int sel_segment(int n) { return ((n + kSelWaves - 1) / kSelWaves + 63) / 64 * 64; }

// A row of at most kRegRowMax elements held in registers: lane l of wave w
// holds elements w * seg + 64 j + l, j < kRegSteps.  Every pass then runs
// without memory reads, its loop fully unrolled into straight-line code.
// Slots past the wave's segment hold a quiet NaN: scores are never NaN (the
// split kernel stores NaN as -inf), a NaN is ignored by fminf / fmaxf, fails
// every comparison and its order-preserving key lies above that of +inf, so
// most passes need no validity test at all.
constexpr int kRegSteps = 32;
constexpr int kRegRowMax = kRegSteps * 64 * kSelWaves;   // 32768

struct RegRow {
  static constexpr bool kWaveSegments = true;   // each() visits wave w's segment in wave w
  float v[kRegSteps];
  int e0;           // this lane's element of step 0
  int steps;        // steps holding elements of this wave's segment (uniform)
  int seg;

  __device__ __forceinline__ int wave_of(uint32_t e) const { return (int)e / seg; }
  __device__ __forceinline__ void load(const float* src, int n) {
    const int w = threadIdx.x >> 6;
    seg = sel_segment(n);
    const int s1 = min(n, w * seg + seg);
    e0 = w * seg + (threadIdx.x & 63);
    steps = __builtin_amdgcn_readfirstlane(s1 > w * seg ? (s1 - w * seg + 63) / 64 : 0);
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j) {
      const int e = e0 + 64 * j;
      const float f = src[min(e, n - 1)];           // in bounds for every lane
      v[j] = e < s1 ? f : __builtin_nanf("");
    }
  }
  template <class F>
  __device__ __forceinline__ void each(F f) const {
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j)
      if (j < steps) f(e0 + 64 * j, v[j] == v[j], v[j]);
  }
  // the scheduling barrier keeps the compiler from computing the lane masks of
  // all steps up front, which would not fit in scalar registers
  template <class F>
  __device__ __forceinline__ void ordered(F f) const {
#pragma unroll
    for (int j = 0; j < kRegSteps; ++j) {
      if (j < steps) f(e0 + 64 * j, v[j] == v[j], v[j]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
};

// A row read from the workspace (rows longer than kRegRowMax).  The loads of
// kSelUnroll elements are issued before any call, so their latencies overlap.
constexpr int kSelUnroll = 8;
struct GlobalRow {
  static constexpr bool kWaveSegments = false;
  const float* vals;
  int n;

  __device__ __forceinline__ int wave_of(uint32_t) const { return 0; }

  template <class F>
  __device__ __forceinline__ void each(F f) const {
    for (int e0 = threadIdx.x; e0 < n; e0 += kSelUnroll * kSelectThreads) {
      float v[kSelUnroll];
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const int e = e0 + u * kSelectThreads;
        v[u] = e < n ? vals[e] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < kSelUnroll; ++u) {
        const int e = e0 + u * kSelectThreads;
        f(e, e < n, v[u]);
      }
    }
  }
  template <class F>
  __device__ __forceinline__ void ordered(F f) const {
    const int seg = sel_segment(n);
    const int s0 = (threadIdx.x >> 6) * seg, s1 = min(n, s0 + seg);
    const int l = threadIdx.x & 63;
    for (int p0 = s0; p0 < s1; p0 += 4 * 64) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + u * 64 + l;
        v[u] = p < s1 ? vals[p] : 0.0f;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int p = p0 + u * 64 + l;
        if (p0 + u * 64 < s1) f(p, p < s1, v[u]);
      }
    }
  }
};

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

typedef LinBucket<kNB> FBucketN;     // linear value buckets (li_bucket.h)
typedef KeyBucket<kNB> UBucketN;     // u32 key buckets of the refining passes

// gathers the (<= kSelSmall) candidates with in(f) into sh.cand_*, then wave 0
// ranks them; the k-th element lands in sh.misc[4..5].  Every element with
// above(f) lies above all candidates, so it is kept.  Where each wave visits
// its own segment (RegRow) the same pass counts them per wave, the ranking wave
// adds the kept candidates to their waves' counts, and the counts of kept
// elements per wave land in sh.misc[kKeptSlot + w] (sh.misc[6] = 1): the
// write needs no counting pass of its own.
template <class Row, class Pred, class Above>
__device__ __forceinline__ void block_gather_rank(SelShared& sh, const Row& row, int r, Pred in,
                                                  Above above) {
  if (threadIdx.x == 0) sh.misc[3] = 0;
  __syncthreads();
  int nab = 0;
  row.each([&](int e, bool valid, float f) {
    const bool take = valid & in(f);
    if constexpr (Row::kWaveSegments) nab += __popcll(ballot(valid & above(f)));
    const uint64_t m = ballot(take);
    if (m != 0) {                          // uniform: one slot reservation per wave
      int base = 0;
      if ((threadIdx.x & 63) == __builtin_ctzll(m)) base = atomicAdd(&sh.misc[3], __popcll(m));
      base = __shfl(base, (int)__builtin_ctzll(m));
      const int slot = base + mbcnt(m);
      if (take && slot < kSelSmall) {
        sh.cand_f[slot] = f;
        sh.cand_e[slot] = (uint32_t)e;
      }
    }
  });
  if constexpr (Row::kWaveSegments) {
    if ((threadIdx.x & 63) == 0) sh.misc[kKeptSlot + (threadIdx.x >> 6)] = nab;
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
    if constexpr (Row::kWaveSegments) {
      const bool kept = (l < m) & ((cf > fb) | ((cf == fb) & (ce <= eb)));
      if (kept) atomicAdd(&sh.misc[kKeptSlot + row.wave_of(ce)], 1);
      if (l == 0) sh.misc[6] = 1;
    }
  }
  __syncthreads();
}

// the r-th entry (index order) whose key equals u; writes fb / eb into sh.misc[4..5]
template <class Row>
__device__ __forceinline__ void block_rth_equal(SelShared& sh, const Row& row, int r, uint32_t u) {
  int cnt = 0;
  row.ordered([&](int, bool valid, float f) { cnt += __popcll(ballot(valid & (f2key(f) == u))); });
  const int before = block_wave_prefix(cnt, sh.misc + 8, nullptr);
  if (before < r && r <= before + cnt) {
    int seen = before;
    row.ordered([&](int p, bool valid, float f) {
      const bool eq = valid & (f2key(f) == u);
      const uint64_t m = ballot(eq);
      // exactly one lane of the whole pass sees itself as the r-th equal entry
      if (eq & (seen + mbcnt(m) == r - 1)) sh.misc[5] = p;
      seen += __popcll(m);
    });
  }
  __syncthreads();
  if (threadIdx.x == 0) sh.misc[4] = __float_as_int(key2f(u));
  __syncthreads();
}

// k-th element of the row in (value desc, index asc) order -> sh.misc[4..5];
// lo / hi are the row's minimum and maximum
template <class Row>
__device__ __forceinline__ void block_kth(SelShared& sh, const Row& row, int k, float lo, float hi) {
  int r = k;
  if (threadIdx.x == 0) sh.misc[6] = 0;     // published by the barriers below
  uint32_t ulo, uhi;
  if (lo < hi) {
    const FBucketN fbk(lo, hi);
    for (int x = threadIdx.x; x < kNB; x += kSelectThreads) sh.hist[x] = 0;
    __syncthreads();
    row.each([&](int, bool valid, float f) { atomicAdd(&sh.hist[hist_slot(valid, fbk(f))], 1u); });
    __syncthreads();
    block_find_bucket(sh, r);
    const uint32_t B = (uint32_t)sh.misc[0];
    const int above = sh.misc[1], cnt = sh.misc[2];
    r -= above;
    __syncthreads();
    if (cnt <= kSelSmall) {
      block_gather_rank(sh, row, r, [&](float f) { return fbk(f) == B; },
                        [&](float f) { return fbk(f) > B; });
      return;
    }
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    row.each([&](int, bool valid, float f) {
      const uint32_t u = f2key(f);
      const bool in = valid & (fbk(f) == B);
      mn = in ? min(mn, u) : mn;
      mx = in ? max(mx, u) : mx;
    });
    ulo = block_min_u(mn, sh.misc + 8);
    uhi = block_max_u(mx, sh.misc + 8);
  } else {
    ulo = uhi = f2key(lo);
  }
  for (;;) {
    if (ulo == uhi) {
      block_rth_equal(sh, row, r, ulo);
      return;
    }
    const UBucketN ubk(ulo, uhi);
    for (int x = threadIdx.x; x < kNB; x += kSelectThreads) sh.hist[x] = 0;
    __syncthreads();
    row.each([&](int, bool valid, float f) {
      const uint32_t u = f2key(f);
      const bool in = valid & (u >= ulo) & (u <= uhi);
      atomicAdd(&sh.hist[hist_slot(in, ubk(u))], 1u);
    });
    __syncthreads();
    block_find_bucket(sh, r);
    const int B = sh.misc[0], above = sh.misc[1], cnt = sh.misc[2];
    r -= above;
    __syncthreads();
    const uint32_t nlo = ulo + ((uint32_t)B << ubk.shift);
    uint32_t nhi = (B == kNB - 1) ? uhi : nlo + ((1u << ubk.shift) - 1u);
    if (nhi > uhi) nhi = uhi;
    if (cnt <= kSelSmall && nlo != nhi) {
      block_gather_rank(
          sh, row, r,
          [&](float f) {
            const uint32_t u = f2key(f);
            return (u >= nlo) & (u <= nhi);
          },
          [&](float f) { return f2key(f) > nhi; });
      return;
    }
    ulo = nlo;
    uhi = nhi;
  }
}

// k-th element and stable, index-ordered write of the top-k of one row.
template <class Row>
__device__ __forceinline__ void select_row(SelShared& sh, const Row& row, int topk, float lo,
                                           float hi, int32_t* oi, float* ov, int ioff) {
  block_kth(sh, row, topk, lo, hi);
  const float fb = __int_as_float(sh.misc[4]);
  const uint32_t eb = (uint32_t)sh.misc[5];
  const bool counted = sh.misc[6] != 0;
  int kept = __builtin_amdgcn_readfirstlane(sh.misc[kKeptSlot + (threadIdx.x >> 6)]);
  __syncthreads();
  if (!counted) {
    kept = 0;
    row.ordered([&](int p, bool valid, float f) {
      kept += __popcll(ballot(valid & ((f > fb) | ((f == fb) & ((uint32_t)p <= eb)))));
    });
  }
  int pos = block_wave_prefix(kept, sh.misc + 8, nullptr);
  const bool has_ov = ov != nullptr;
  row.ordered([&](int p, bool valid, float f) {
    const bool keep = valid & ((f > fb) | ((f == fb) & ((uint32_t)p <= eb)));
    const uint64_t m = ballot(keep);
    const int o = pos + mbcnt(m);
    const bool st = keep & (o < topk);     // bounded whatever the data
    if (st) oi[o] = p + ioff;
    if (st & has_ov) ov[o] = f;
    pos += __popcll(m);
  });
}

__global__ __launch_bounds__(kSelectThreads) void select_kernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  SelShared& sh = *reinterpret_cast<SelShared*>(smem);
  // The grid is one workgroup per (batch, row): exactly batch * S1max of them,
  // so b < batch.  Everything the row needs that
  // does not come from the metadata (its lengths from the call's arguments, the
  // first 64 segment ranges, the index offset) is loaded before the metadata
  // check, so that these latencies overlap instead of queueing one after the
  // other; the row itself follows as soon as its length is known.
  const int r = blockIdx.x;
  const int b = r / a.s1max, i = r - (r / a.s1max) * a.s1max;
  const int tid = threadIdx.x;
  const int4 br = batch_lengths(a, b);
  const float* mm = a.seg_mm + (int64_t)r * a.seg_mm_stride * 2;
  const int j0 = tid & 63;
  const bool in0 = j0 < a.seg_mm_stride;
  const float mm_lo0 = mm[2 * (in0 ? j0 : 0)], mm_hi0 = mm[2 * (in0 ? j0 : 0) + 1];
  const int ioff = index_offset(a, b);
  const int lim = row_limit(a, b, i, br.y, br.w);
  if (!check_meta(a)) return;
  if (i >= br.y) return;
  const int topk = a.topk;
  const int64_t tok = (int64_t)br.x + i;
  int32_t* oi = a.out_idx + tok * topk;
  float* ov = a.out_val ? a.out_val + tok * topk : nullptr;
  const float* src = a.ws + ((int64_t)b * a.s1max + i) * a.ws_row_stride;

  if (lim <= topk) {
    for (int e = tid; e < topk; e += kSelectThreads) {
      if (e < lim) {
        oi[e] = e + ioff;
        if (ov) ov[e] = src[e];
      } else {
        oi[e] = -1;
        if (ov) ov[e] = -__builtin_inff();
      }
    }
    return;
  }
  // the row's range from its segments' (min, max), reduced by every wave on
  // its own (no barrier), with the row's own loads in flight
  const int chunk = reinterpret_cast<const MetaHeader*>(a.meta)->chunk;
  const int nseg = (lim + chunk - 1) / chunk;
  auto range = [&](float& lo, float& hi) __attribute__((always_inline)) {
    float mn = j0 < nseg ? mm_lo0 : __builtin_inff();
    float mx = j0 < nseg ? mm_hi0 : -__builtin_inff();
    for (int j = j0 + 64; j < nseg; j += 64) {
      mn = fminf(mn, mm[2 * j]);
      mx = fmaxf(mx, mm[2 * j + 1]);
    }
    lo = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_min_f(mn))));
    hi = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(wave_max_f(mx))));
  };
  float lo, hi;
  if (lim <= kRegRowMax) {
    RegRow row;
    row.load(src, lim);
    range(lo, hi);
    select_row(sh, row, topk, lo, hi, oi, ov, ioff);
  } else {
    range(lo, hi);
    const GlobalRow row{src, lim};
    select_row(sh, row, topk, lo, hi, oi, ov, ioff);
  }
}

template <int QK, int MB, int WT, int KL>
hipError_t launch_split(const KArgs& a, int grid, hipStream_t s) {
  constexpr size_t lds = (size_t)kDecodeWaves * kPipeKeys * Mma<QK>::RB;   // one K tile per wave
  hipLaunchKernelGGL((split_kernel<QK, MB, WT, KL>), dim3(grid), dim3(kDecodeWaves * 64), lds, s, a);
  return hipGetLastError();
}

template <int QK, int MB, int WT>
hipError_t launch_split_p(const KArgs& a, int kl, int grid, hipStream_t s) {
  switch (kl) {
    case KL_CONTIG: return launch_split<QK, MB, WT, KL_CONTIG>(a, grid, s);
    case KL_PAGED: return launch_split<QK, MB, WT, KL_PAGED>(a, grid, s);
    default: return launch_split<QK, MB, WT, KL_PAGED_TILE>(a, grid, s);
  }
}

template <int QK, int MB>
hipError_t launch_split_w(const KArgs& a, int w_dtype, int kl, int grid, hipStream_t s) {
  return w_dtype == DT_FP32 ? launch_split_p<QK, MB, DT_FP32>(a, kl, grid, s)
                            : launch_split_p<QK, MB, DT_BF16>(a, kl, grid, s);
}

template <int QK>
hipError_t launch_split_mb(const KArgs& a, int w_dtype, int mblocks, int kl, int grid,
                           hipStream_t s) {
  return mblocks == 1 ? launch_split_w<QK, 1>(a, w_dtype, kl, grid, s)
                      : launch_split_w<QK, 2>(a, w_dtype, kl, grid, s);
}

}  // namespace

size_t select_shared_bytes() { return sizeof(SelShared); }

hipError_t launch_decode(const KArgs& a, int qk_dtype, int w_dtype, int mblocks, int kl,
                         int grid, hipStream_t s) {
  switch (qk_dtype) {
    case DT_BF16: return launch_split_mb<DT_BF16>(a, w_dtype, mblocks, kl, grid, s);
    case DT_FP16: return launch_split_mb<DT_FP16>(a, w_dtype, mblocks, kl, grid, s);
    case DT_FP8: return launch_split_mb<DT_FP8>(a, w_dtype, mblocks, kl, grid, s);
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
