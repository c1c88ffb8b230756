// Prefill kernels: scores of a block of query rows against every visible key,
// fused with an exact top-k per row, so the score matrix never leaves the chip.
//
// Score (npu_lightning_indexer_pto page, formula under "功能说明"; lightning_indexer
// page, "Function" steps 1-3): I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:]).
// The Q.K^T tile is an MFMA contraction with heads on M and keys on N; ReLU, the
// weights and the head sum run on the fp32 accumulators in registers.  One wave
// owns one query row; the workgroup shares each 64-key K tile through LDS.
//
// Top-k (lightning_indexer page, step 3; -1 / -inf padding from its Constraints):
//  - dense kernel (rows of at most `dcap` visible keys): 4 waves, each keeps its
//    row's scores in LDS, indexed by key; rows with no more visible keys than k
//    are written straight to the output, the others pick their k-th element with
//    the exact bucket select and write the kept keys in ascending key order.  At
//    <= 80 KiB of LDS two workgroups share a CU, so one workgroup's MFMAs run
//    while the other is in its epilogue, select or output phase;
//  - streaming kernel (longer rows): 4 waves, each keeps a list of up to `cap`
//    (score, key) candidates in ascending key order.  A key enters when it beats
//    the running threshold; a full list is cut back to exactly k entries by the
//    exact select (ties to smaller keys) and the threshold rises to the k-th
//    score.  Keys arrive in increasing order, so a later key never wins a tie.
#include "li_common_kernels.h"
#include "li_pipe.h"
#include "li_select.h"

namespace li {

namespace {

// -0 -> +0, and NaN (only possible from NaN inputs) -> -inf, so that every
// stored score is ordered and the exact select's counting invariant holds.
__device__ inline float canon(float f) {
  if (f == 0.0f) return 0.0f;
  return f != f ? -__builtin_inff() : f;
}
// The same in two VALU ops instead of four: f is an arithmetic result, so a
// NaN is quiet and max(f, -inf) returns -inf for it; adding +0 then turns -0
// into +0 (round to nearest).
__device__ inline float canon2(float f) { return __builtin_fmaxf(f, -__builtin_inff()) + 0.0f; }

// Writes the top-k of a score row in ascending key order, given its k-th element.
// vals: LDS scores; idx: LDS keys or nullptr (key = position).  At most topk
// entries are written whatever the data; each index plus ioff (the batch's
// output index offset).
__device__ inline void write_kept(const float* vals, const uint32_t* idx, int n, float fb,
                                  uint32_t eb, int32_t* oi, float* ov, int topk, int ioff) {
  const int l = lane_id();
  int kept = 0;
  for (int p0 = 0; p0 < n; p0 += 64) {
    const int p = p0 + l;
    float f = 0.0f;
    uint32_t e = 0;
    bool keep = false;
    if (p < n) {
      f = vals[p];
      e = idx ? idx[p] : (uint32_t)p;
      keep = f > fb || (f == fb && e <= eb);
    }
    const uint64_t m = ballot(keep);
    if (keep) {
      const int pos = kept + mbcnt(m);
      if (pos < topk) {
        oi[pos] = (int32_t)e + ioff;
        if (ov) ov[pos] = f;
      }
    }
    kept += __popcll(m);
  }
}

// write_kept for a row in global memory, the index of entry p being p.
__device__ inline void write_kept_row(const float* vals, int n, float fb, uint32_t eb,
                                      int32_t* oi, float* ov, int topk, int ioff) {
  int kept = 0;
  row_pass(vals, n, [&](int p, bool valid, float f) __attribute__((always_inline)) {
    const bool keep = valid && (f > fb || (f == fb && (uint32_t)p <= eb));
    const uint64_t m = ballot(keep);
    if (keep) {
      const int pos = kept + mbcnt(m);
      if (pos < topk) {
        oi[pos] = p + ioff;
        if (ov) ov[pos] = f;
      }
    }
    kept += __popcll(m);
  });
}

__device__ inline void write_padding(int n, int topk, int32_t* oi, float* ov) {
  for (int e = n + lane_id(); e < topk; e += 64) {
    oi[e] = -1;
    if (ov) ov[e] = -__builtin_inff();
  }
}

// Output of a wave's candidate list (key order): its top-k, streamed straight
// from the list once the k-th element is known, then the padding.
__device__ inline void write_list_topk(const float* listF, const uint32_t* listI, int count,
                                       int topk, uint32_t* hist, uint32_t* scr, int32_t* oi,
                                       float* ov, int ioff) {
  const int lane = lane_id();
  if (count > topk) {
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    for (int p = lane; p < count; p += 64) {
      const float f = listF[p];
      vmin = fminf(vmin, f);
      vmax = fmaxf(vmax, f);
    }
    float fb;
    uint32_t eb;
    wave_kth(listF, listI, count, topk, wave_min_f(vmin), wave_max_f(vmax), hist, scr, fb, eb);
    write_kept(listF, listI, count, fb, eb, oi, ov, topk, ioff);
    return;
  }
  for (int e = lane; e < count; e += 64) {
    oi[e] = (int32_t)listI[e] + ioff;
    if (ov) ov[e] = listF[e];
  }
  write_padding(count, topk, oi, ov);
}

// ---------------------------------------------------------------------------
// dense kernel: 4 rows per workgroup, every score of a row kept densely, in
// LDS (G = false) or, for rows too long for LDS, in a global workspace row per
// wave of each resident workgroup (G = true; the grid is then one workgroup per
// slot, two per CU, each walking the work list with a stride of the grid).
// ---------------------------------------------------------------------------
template <int QK, int MB, int WT, int KL, bool G>
__device__ __forceinline__ void dense_item(const KArgs& a, int it, unsigned char* smem) {
  typedef Mma<QK> M;
  typedef typename M::frag F;
  constexpr int NT = kDenseWaves * 64;
  constexpr int TILE = kPipeKeys * M::RB;
  // [0, R0): two K tiles and the descale slots during the score loop, the
  // per-wave select scratch afterwards; then (G = false) the score rows
  constexpr int DSC = 2 * TILE;                      // descale slots (fp8 only)
  constexpr int R0a = DSC + (QK == DT_FP8 ? kDscSlots * 32 * 4 : 0);
  constexpr int SCR = G ? kWideScratch : kDenseScratch;
  constexpr int R0 = R0a > kDenseWaves * SCR ? R0a : kDenseWaves * SCR;
  float* dsc_lds = reinterpret_cast<float*>(smem + DSC);

  // opaque per item: lane-derived offsets are recomputed in each item instead of
  // being hoisted out of the item loop and held through the score loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int topk = a.topk;
  float* row = G ? a.ws + ((int64_t)blockIdx.x * kDenseWaves + wave) * a.ws_row_stride
                 : reinterpret_cast<float*>(smem + R0) + wave * a.dcap;
  const int4 item = reinterpret_cast<const int4*>(a.meta + a.off_items)[it];
  const int b = item.x, q0 = item.y, nrows = item.z;
  const int4 br = batch_rec(a, b);               // q_off, s1, k_off, s2
  const int ioff = index_offset(a, b);

  const bool has_row = wave < nrows;
  const int i = q0 + wave;
  const int lim = has_row ? row_limit(a, b, i, br.y, br.w) : 0;
  const int kend = row_limit(a, b, q0 + nrows - 1, br.y, br.w);
  const int ntiles = (kend + kPipeKeys - 1) / kPipeKeys;
  const int64_t tok = (int64_t)br.x + i;
  const bool direct = lim <= topk;
  int32_t* oi = a.out_idx + tok * topk;
  float* ov = a.out_val ? a.out_val + tok * topk : nullptr;

  // fp8 tiles are half the registers: four in flight hide more of the L2 / MALL latency
  constexpr int D = QK == DT_FP8 ? 4 : kStageDepth;
  PipeStage<QK, KL, NT, D, G> st;
  st.prefetch_table(a, b, 0);
  F qf[MB][M::KSTEPS];
  float wv[MB][16];
  // the query goes through LDS (coalesced loads); each wave's staging area
  // overlaps the K tiles and the rows, so all waves finish with it first
  if (has_row) load_query<QK, MB, WT, true>(a, tok, lane, qf, wv, smem + wave * q_stage_bytes<QK>());
  else zero_query<QK, MB>(qf, wv);
  settle_loads();
  __syncthreads();

  // results of tile t (descaled): lanes 0-31 carry keys t*32 + lane, lanes
  // 32-63 the same scores again.  Every row's scores go to its row (the rows
  // that need no select are copied out after the loop), so a step's memory
  // operations never depend on the row: a data-dependent global store inside
  // the loop would make every wait for the K ring wait for it as well.  The
  // row's minimum and maximum are tracked here.
  float vmin = __builtin_inff(), vmax = -__builtin_inff();
  auto emit = [&](int t, float tot) {
    const int s = t * kPipeKeys + (lane & 31);
    const bool in = lane < 32 && s < lim;
    // Fewer VALU ops pay off where the rows live in global memory; with LDS
    // rows (up to 4096 keys) the longer forms measure faster (schedule effect).
    const float f = G ? canon2(tot) : canon(tot);
    if constexpr (G) {
      // every lane stores (lanes 32-63 repeat lanes 0-31); keys past lim land
      // below the row stride, in slots that are never read
      row[s] = f;
    } else {
      if (in) row[s] = f;
    }
    if constexpr (G) {
      // f is never NaN: a compare and a select each, no operand quieting
      vmin = (in & (f < vmin)) ? f : vmin;
      vmax = (in & (f > vmax)) ? f : vmax;
    } else {
      vmin = in ? fminf(vmin, f) : vmin;
      vmax = in ? fmaxf(vmax, f) : vmax;
    }
  };

  f32x16 accA[MB], accB[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accA[mb] = f32x16{};
    accB[mb] = f32x16{};
  }
  if (ntiles > 0) {
    st.template load<0>(a, b, br.z, 0, kend, tid);
    st.template load<1>(a, b, br.z, kPipeKeys, kend, tid);
    if constexpr (D > 2) {
      st.template load<2 % D>(a, b, br.z, 2 * kPipeKeys, kend, tid);
      st.template load<3 % D>(a, b, br.z, 3 * kPipeKeys, kend, tid);
    }
    st.template store<0>(smem, tid);
    st.template store_dsc<0>(dsc_lds, tid);
  }
  __syncthreads();

  // Step t (ring set S = t % D): store tile t+1 into the other LDS buffer, load
  // tile t+D into set S, MFMAs of tile t into `cur` interleaved with the
  // epilogue of tile t-1 from `prev`, then tile t-2's scores are written: they
  // are a step old, so the write never waits on the epilogue's latency.
  float pend = 0.0f;                       // descaled scores of tile t-1, not yet written
  auto step = [&](auto set, int t, f32x16 (&cur)[MB], const f32x16 (&prev)[MB]) __attribute__((always_inline)) {
    constexpr int S = decltype(set)::value;
    // set S (tile t) went to LDS in the previous step: refill it first, so
    // the wait for tile t+1 below leaves D-1 tiles in flight
    st.template load<S>(a, b, br.z, (t + D) * kPipeKeys, kend, tid);
    // tile t's fragments are read before tile t+1 is stored, so that the
    // MFMAs' reads do not queue behind the stores in the LDS
    F kb[M::KSTEPS];
    read_tile_frags<QK>(smem + (t & 1) * TILE, lane, kb);
    st.template store<(S + 1) % D>(smem + ((t + 1) & 1) * TILE, tid);
    st.template store_dsc<(S + 1) % D>(dsc_lds + ((t + 1) & (kDscSlots - 1)) * 32, tid);
    const float ds = QK == DT_FP8 ? dsc_lds[((t - 1) & (kDscSlots - 1)) * 32 + (lane & 31)] : 1.0f;
    __builtin_amdgcn_s_setprio(2);
    mma_tile<QK, MB>(qf, kb, cur);
    const float prev_score = block_score<MB>(prev, wv);
    // the per-key paged addressing leaves no room for every fragment at once
    pipe_schedule<QK, MB, KL != KL_PAGED>();
    __builtin_amdgcn_s_setprio(1);
    if (t > 1) emit(t - 2, pend);
    pend = QK == DT_FP8 ? prev_score * ds : prev_score;
    __syncthreads();
  };
  // Full groups of 4 steps (two accumulator sets x ring) run unconditionally, so
  // every step issues the same loads and the waits stay static counts; the last
  // 0-3 tiles follow.
  // Issue priority: a wave in its MFMA stretch first (2), then a wave in the
  // score loop (1), then a wave loading its query or selecting (0).  The SIMD's
  // other wave, from the other workgroup on the CU, is often in a different
  // phase; this keeps the matrix core fed from whichever wave has MFMAs ready.
  int t = 0;
  __builtin_amdgcn_s_setprio(1);
  for (; t + 4 <= ntiles; t += 4) {
    step(IntC<0>(), t, accA, accB);
    step(IntC<1>(), t + 1, accB, accA);
    step(IntC<2 % D>(), t + 2, accA, accB);
    step(IntC<3 % D>(), t + 3, accB, accA);
  }
  if (t < ntiles) step(IntC<0>(), t, accA, accB);
  if (t + 1 < ntiles) step(IntC<1>(), t + 1, accB, accA);
  if (t + 2 < ntiles) step(IntC<2 % D>(), t + 2, accA, accB);
  if (ntiles > 0) {
    const int last = ntiles - 1;
    const float ds = QK == DT_FP8 ? dsc_lds[(last & (kDscSlots - 1)) * 32 + (lane & 31)] : 1.0f;
    const float sc = (last & 1) ? block_score<MB>(accB, wv) : block_score<MB>(accA, wv);
    if (last > 0) emit(last - 1, pend);
    emit(last, QK == DT_FP8 ? sc * ds : sc);
  }
  __syncthreads();                         // the tile area becomes select scratch
  __builtin_amdgcn_s_setprio(0);
  if (!has_row) return;
  if (direct) {
    // every visible key is kept: the row in key order, then the padding
    if (lim > 0) {
      row_pass(row, lim, [&](int p, bool valid, float f) __attribute__((always_inline)) {
        if (valid) {
          oi[p] = p + ioff;
          if (ov) ov[p] = f;
        }
      });
    }
    write_padding(lim, topk, oi, ov);
    return;
  }
  float fb;
  uint32_t eb;
  const float lo = wave_min_f(vmin), hi = wave_max_f(vmax);
  if constexpr (G) {
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + wave * kWideScratch);
    uint32_t* scr = hist + kWideBuckets;
    if (!wave_topk_row_call<kWideBuckets>(row, lim, topk, lo, hi, hist, scr, oi, ov, ioff)) {
      wave_kth(row, nullptr, lim, topk, lo, hi, scr + 2 * kSelSmall, scr, fb, eb);
      write_kept_row(row, lim, fb, eb, oi, ov, topk, ioff);
    }
  } else {
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + wave * kDenseScratch);
    uint32_t* scr = hist + kLdsBuckets;
    if (!wave_topk_row<kLdsBuckets>(row, lim, topk, lo, hi, hist, scr, oi, ov, ioff)) {
      wave_kth(row, nullptr, lim, topk, lo, hi, hist, scr, fb, eb);
      write_kept(row, nullptr, lim, fb, eb, oi, ov, topk, ioff);
    }
  }
}

template <int QK, int MB, int WT, int KL, bool G>
__global__ __launch_bounds__(kDenseWaves * 64, 2) void dense_kernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if (!check_meta(a)) return;
  const int n_items = reinterpret_cast<const MetaHeader*>(a.meta)->n_items;
  if constexpr (!G) {
    if ((int)blockIdx.x < n_items) dense_item<QK, MB, WT, KL, G>(a, blockIdx.x, smem);
  } else {
    for (int it = blockIdx.x; it < n_items; it += gridDim.x) {
      // the previous item's select scratch overlaps the K tiles
      if (it != (int)blockIdx.x) __syncthreads();
      dense_item<QK, MB, WT, KL, G>(a, it, smem);
    }
  }
}

// ---------------------------------------------------------------------------
// streaming kernels: 4 rows per workgroup, a bounded candidate list per row
// ---------------------------------------------------------------------------
// stream_shared_kernel (bf16 / fp16 keys): the dense kernel's pipeline (32-key
// tiles shared by the workgroup, double-buffered in LDS, one barrier per tile,
// MFMAs of tile t interleaved with the epilogue of tile t-1); instead of a full
// score row each wave keeps a candidate list.  Sharing the tile keeps the LDS
// traffic at one tile write per step, which 256-byte key rows need.
template <int QK, int MB, int WT, int KL>
__global__ __launch_bounds__(kStreamWaves * 64, 1) void stream_shared_kernel(KArgs a) {
  typedef Mma<QK> M;
  typedef typename M::frag F;
  constexpr int NT = kStreamWaves * 64;
  constexpr int TILE = kPipeKeys * M::RB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  if (!check_meta(a)) return;
  const MetaHeader* hdr = reinterpret_cast<const MetaHeader*>(a.meta);
  if ((int)blockIdx.x >= hdr->n_items) return;
  const int4 item = reinterpret_cast<const int4*>(a.meta + a.off_items)[blockIdx.x];
  const int b = item.x, q0 = item.y, nrows = item.z;
  const int4 br = batch_rec(a, b);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int cap = a.cap, topk = a.topk;
  const int ioff = index_offset(a, b);

  // LDS: two K tiles, the descale slots, the per-wave select scratch, the lists
  constexpr int SCR = 2 * TILE + (QK == DT_FP8 ? kDscSlots * 32 * 4 : 0);
  float* dsc_lds = reinterpret_cast<float*>(smem + 2 * TILE);
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + SCR + wave * kWaveScratch);
  uint32_t* scr = hist + 256;
  float* listF = reinterpret_cast<float*>(smem + SCR + kStreamWaves * kWaveScratch) + wave * cap;
  uint32_t* listI = reinterpret_cast<uint32_t*>(listF) + kStreamWaves * cap;

  const bool has_row = wave < nrows;
  const int i = q0 + wave;
  const int lim = has_row ? row_limit(a, b, i, br.y, br.w) : 0;
  const int kend = row_limit(a, b, q0 + nrows - 1, br.y, br.w);
  const int ntiles = (kend + kPipeKeys - 1) / kPipeKeys;
  const int64_t tok = (int64_t)br.x + i;

  constexpr int D = kStreamStageDepth;
  PipeStage<QK, KL, NT, D> st;
  st.prefetch_table(a, b, 0);
  F qf[MB][M::KSTEPS];
  float wv[MB][16];
  if (has_row) load_query<QK, MB, WT>(a, tok, lane, qf, wv);
  else zero_query<QK, MB>(qf, wv);
  settle_loads();

  int count = 0;                           // candidates in this wave's list (wave-uniform)
  // A key enters the list if it beats the k-th candidate: score above `thr`
  // (keys arrive in increasing order, so a later key never wins a tie).  Until
  // the first cut there is no k-th candidate and every key enters (incl).
  float thr = -__builtin_inff();
  bool incl = true;

  // Cuts the list back to exactly k entries (in key order, in place); the
  // threshold rises to the k-th score.  Called between groups of tiles only,
  // so that the insertions below never need it.
  auto compact = [&]() __attribute__((always_inline)) {
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    for (int p = lane; p < count; p += 64) {
      const float f = listF[p];
      vmin = fminf(vmin, f);
      vmax = fmaxf(vmax, f);
    }
    float fb;
    uint32_t eb;
    wave_kth(listF, listI, count, topk, wave_min_f(vmin), wave_max_f(vmax), hist, scr, fb, eb);
    int kept = 0;
    for (int p0 = 0; p0 < count; p0 += 64) {
      const int p = p0 + lane;
      float f = 0.0f;
      uint32_t e = 0;
      bool keep = false;
      if (p < count) {
        f = listF[p];
        e = listI[p];
        keep = f > fb || (f == fb && e <= eb);
      }
      const uint64_t km = ballot(keep);
      wave_sync();
      if (keep) {
        const int pos = kept + mbcnt(km);
        if (pos < cap) {
          listF[pos] = f;
          listI[pos] = e;
        }
      }
      kept += __popcll(km);
      wave_sync();
    }
    count = kept < topk ? kept : topk;     // exactly topk for ordered scores
    thr = fb;
    incl = false;
  };

  // results of tile t (descaled): lanes 0-31 carry keys t*32 + lane.  The list
  // has room for them (count <= cap - 32).
  auto emit = [&](int t, float tot) __attribute__((always_inline)) {
    const int s = t * kPipeKeys + lane;
    tot = canon(tot);
    const bool want = (lane < 32) & (s < lim) & (incl ? tot >= thr : tot > thr);
    const uint64_t m = ballot(want);
    if (m != 0) {                          // uniform
      const int pos = count + mbcnt(m);
      if (want & (pos < cap)) {            // always room; bounded whatever the data
        listF[pos] = tot;
        listI[pos] = (uint32_t)s;
      }
      count += __popcll(m);
    }
  };

  f32x16 accA[MB], accB[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accA[mb] = f32x16{};
    accB[mb] = f32x16{};
  }
  if (ntiles > 0) {
    st.template load<0>(a, b, br.z, 0, kend, tid);
    st.template load<1>(a, b, br.z, kPipeKeys, kend, tid);
    if constexpr (D > 2) {
      st.template load<2 % D>(a, b, br.z, 2 * kPipeKeys, kend, tid);
      st.template load<3 % D>(a, b, br.z, 3 * kPipeKeys, kend, tid);
    }
    st.template store<0>(smem, tid);
    st.template store_dsc<0>(dsc_lds, tid);
  }
  __syncthreads();

  // Step t (ring set S = t % D): store tile t+1 into the other LDS buffer, load
  // tile t+D into set S, MFMAs of tile t into `cur` interleaved with the
  // epilogue of tile t-1 from `prev`, then tile t-2's candidates: their scores
  // are a step old, so the insertion never waits on the epilogue's latency.
  float pend = 0.0f;                       // descaled scores of tile t-1, not yet inserted
  auto step = [&](auto set, int t, f32x16 (&cur)[MB], const f32x16 (&prev)[MB])
                  __attribute__((always_inline)) {
    constexpr int S = decltype(set)::value;
    // set S (tile t) went to LDS in the previous step: refill it first, so
    // the wait for tile t+1 below leaves D-1 tiles in flight
    st.template load<S>(a, b, br.z, (t + D) * kPipeKeys, kend, tid);
    st.template store<(S + 1) % D>(smem + ((t + 1) & 1) * TILE, tid);
    st.template store_dsc<(S + 1) % D>(dsc_lds + ((t + 1) & (kDscSlots - 1)) * 32, tid);
    F kb[M::KSTEPS];
    read_tile_frags<QK>(smem + (t & 1) * TILE, lane, kb);
    // tile t-1's descales (fp8), read early so the latency hides behind the MFMAs
    const float ds = QK == DT_FP8 ? dsc_lds[((t - 1) & (kDscSlots - 1)) * 32 + (lane & 31)] : 1.0f;
    mma_tile<QK, MB>(qf, kb, cur);
    const float prev_score = block_score<MB>(prev, wv);
    pipe_schedule<QK, MB>();
    if (t > 1) emit(t - 2, pend);
    pend = QK == DT_FP8 ? prev_score * ds : prev_score;
    __syncthreads();
  };
  // A group of 4 steps, or the last 0-3 steps and the two final emits, insert
  // at most 5 * 32 keys: the list is cut back before them if there might not be
  // room.
  // Full groups run unconditionally (static waits, see the dense kernel); the
  // last 0-3 tiles follow.
  int t = 0;
  for (; t + 4 <= ntiles; t += 4) {
    if (count > cap - 5 * kPipeKeys) compact();   // cap >= k + 5 * 32: count > k here
    step(IntC<0>(), t, accA, accB);
    step(IntC<1>(), t + 1, accB, accA);
    step(IntC<2 % D>(), t + 2, accA, accB);
    step(IntC<3 % D>(), t + 3, accB, accA);
  }
  if (count > cap - 5 * kPipeKeys) compact();
  if (t < ntiles) step(IntC<0>(), t, accA, accB);
  if (t + 1 < ntiles) step(IntC<1>(), t + 1, accB, accA);
  if (t + 2 < ntiles) step(IntC<2 % D>(), t + 2, accA, accB);
  if (ntiles > 0) {
    const int last = ntiles - 1;
    const float ds = QK == DT_FP8 ? dsc_lds[(last & (kDscSlots - 1)) * 32 + (lane & 31)] : 1.0f;
    const float sc = (last & 1) ? block_score<MB>(accB, wv) : block_score<MB>(accA, wv);
    if (last > 0) emit(last - 1, pend);
    emit(last, QK == DT_FP8 ? sc * ds : sc);
  }

  if (!has_row) return;
  int32_t* oi = a.out_idx + tok * topk;
  float* ov = a.out_val ? a.out_val + tok * topk : nullptr;
  write_list_topk(listF, listI, count, topk, hist, scr, oi, ov, ioff);
}

// stream_kernel (fp8 keys; every key dtype when a large topk leaves room for
// two rows per workgroup, W = 2): each wave owns one row and works alone, with no
// workgroup barrier: it streams its own visible keys through a 4-deep register
// ring of 32-key tiles (coalesced loads), a wave-private LDS tile for the MFMA
// operand layout, and its MFMAs interleaved with the epilogue of the previous
// tile.  A wave whose
// list needs cutting back, or whose row is shorter, never holds up the others;
// the 128-byte key rows keep the four private tile copies within the LDS
// bandwidth the MFMAs leave.
template <int QK, int MB, int WT, int KL, int W>
__global__ __launch_bounds__(W * 64, 1) void stream_kernel(KArgs a) {
  typedef Mma<QK> M;
  typedef typename M::frag F;
  constexpr int D = kStreamStageDepth;
  constexpr int TILE = kPipeKeys * M::RB;
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];

  if (!check_meta(a)) return;
  const MetaHeader* hdr = reinterpret_cast<const MetaHeader*>(a.meta);
  if ((int)blockIdx.x >= hdr->n_items) return;
  const int4 item = reinterpret_cast<const int4*>(a.meta + a.off_items)[blockIdx.x];
  const int b = item.x, q0 = item.y, nrows = item.z;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wave >= nrows) return;
  const int4 br = batch_rec(a, b);
  const int cap = a.cap, topk = a.topk;
  const int ioff = index_offset(a, b);
  const int i = q0 + wave;
  const int lim = row_limit(a, b, i, br.y, br.w);
  const int64_t tok = (int64_t)br.x + i;
  int32_t* oi = a.out_idx + tok * topk;
  float* ov = a.out_val ? a.out_val + tok * topk : nullptr;

  // LDS: per-wave K tiles, per-wave select scratch, per-wave lists
  unsigned char* tile = smem + wave * TILE;
  uint32_t* hist = reinterpret_cast<uint32_t*>(smem + W * TILE + wave * kWaveScratch);
  uint32_t* scr = hist + 256;
  float* listF = reinterpret_cast<float*>(smem + W * (TILE + kWaveScratch)) + wave * cap;
  uint32_t* listI = reinterpret_cast<uint32_t*>(listF) + W * cap;

  if (lim == 0) {
    write_padding(0, topk, oi, ov);
    return;
  }
  PipeStage<QK, KL, 64, D> st;
  st.prefetch_table(a, b, 0);
  F qf[MB][M::KSTEPS];
  float wv[MB][16];
  load_query<QK, MB, WT>(a, tok, lane, qf, wv);

  int count = 0;                           // candidates in the list (wave-uniform)
  // A key enters the list if it beats the k-th candidate: score above `thr`
  // (keys arrive in increasing order, so a later key never wins a tie).  Until
  // the first cut there is no k-th candidate and every key enters (incl).
  float thr = -__builtin_inff();
  bool incl = true;

  // Cuts the list back to exactly k entries (in key order, in place); the
  // threshold rises to the k-th score.  Called between groups of tiles only,
  // so that the insertions below never need it.
  auto compact = [&]() __attribute__((always_inline)) {
    float vmin = __builtin_inff(), vmax = -__builtin_inff();
    for (int p = lane; p < count; p += 64) {
      const float f = listF[p];
      vmin = fminf(vmin, f);
      vmax = fmaxf(vmax, f);
    }
    float fb;
    uint32_t eb;
    wave_kth(listF, listI, count, topk, wave_min_f(vmin), wave_max_f(vmax), hist, scr, fb, eb);
    int kept = 0;
    for (int p0 = 0; p0 < count; p0 += 64) {
      const int p = p0 + lane;
      float f = 0.0f;
      uint32_t e = 0;
      bool keep = false;
      if (p < count) {
        f = listF[p];
        e = listI[p];
        keep = f > fb || (f == fb && e <= eb);
      }
      const uint64_t km = ballot(keep);
      wave_sync();
      if (keep) {
        const int pos = kept + mbcnt(km);
        if (pos < cap) {
          listF[pos] = f;
          listI[pos] = e;
        }
      }
      kept += __popcll(km);
      wave_sync();
    }
    count = kept < topk ? kept : topk;     // exactly topk for ordered scores
    thr = fb;
    incl = false;
  };

  // results of tile t (descaled): lanes 0-31 carry keys t*32 + lane.  The list
  // has room for them (count <= cap - 32).
  auto emit = [&](int t, float tot) __attribute__((always_inline)) {
    const int s = t * kPipeKeys + lane;
    tot = canon(tot);
    const bool want = (lane < 32) & (s < lim) & (incl ? tot >= thr : tot > thr);
    const uint64_t m = ballot(want);
    if (m != 0) {                          // uniform
      const int pos = count + mbcnt(m);
      if (want & (pos < cap)) {            // always room; bounded whatever the data
        listF[pos] = tot;
        listI[pos] = (uint32_t)s;
      }
      count += __popcll(m);
    }
  };

  const int ntiles = (lim + kPipeKeys - 1) / kPipeKeys;
  f32x16 accA[MB], accB[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accA[mb] = f32x16{};
    accB[mb] = f32x16{};
  }
  static_for<D>([&](auto set) {
    constexpr int S = decltype(set)::value;
    st.template load<S>(a, b, br.z, S * kPipeKeys, lim, lane);
  });

  // Step t (ring set S = t % D): tile t from set S into the wave's LDS tile,
  // refill set S with tile t + D, MFMAs of tile t into one accumulator set
  // interleaved with the epilogue of tile t - 1 from the other, then tile t-2's
  // candidates: their scores are a step old, so the insertion never waits on
  // the epilogue's latency.
  float dcur = 1.0f;                       // descales (fp8) of tile t, then t-1
  float pend = 0.0f;                       // descaled scores of tile t-1, not yet inserted
  auto step = [&](auto set, int t) __attribute__((always_inline)) {
    constexpr int S = decltype(set)::value;
    f32x16(&cur)[MB] = (S & 1) ? accB : accA;
    f32x16(&prev)[MB] = (S & 1) ? accA : accB;
    st.template store<S>(tile, lane);
    const float dprev = dcur;
    dcur = st.dsc[S];
    st.template load<S>(a, b, br.z, (t + D) * kPipeKeys, lim, lane);
    wave_sync();
    F kb[M::KSTEPS];
    read_tile_frags<QK>(tile, lane, kb);
    mma_tile<QK, MB>(qf, kb, cur);
    const float prev_score = block_score<MB>(prev, wv);
    pipe_schedule<QK, MB>();
    if (t > 1) emit(t - 2, pend);
    pend = QK == DT_FP8 ? prev_score * dprev : prev_score;
    wave_sync();
  };
  // Full groups of D steps run unconditionally (every step issues the same
  // loads: static waits, the ring never drains); the last tiles follow one by
  // one.  A group, or the tail with the two final insertions, adds at most
  // 5 * 32 keys: the list is cut back before them if there might not be room.
  int t = 0;
  for (; t + D <= ntiles; t += D) {
    if (count > cap - 5 * kPipeKeys) compact();   // cap >= k + 5 * 32: count > k here
    static_for<D>([&](auto set) { step(set, t + decltype(set)::value); });
  }
  if (count > cap - 5 * kPipeKeys) compact();
  static_for<D - 1>([&](auto set) {
    if (t + decltype(set)::value < ntiles) step(set, t + decltype(set)::value);
  });
  {
    const int last = ntiles - 1;
    const float sc = (last & 1) ? block_score<MB>(accB, wv) : block_score<MB>(accA, wv);
    if (last > 0) emit(last - 1, pend);
    emit(last, QK == DT_FP8 ? sc * dcur : sc);
  }

  write_list_topk(listF, listI, count, topk, hist, scr, oi, ov, ioff);
}

template <class K>
hipError_t launch_kernel(K fn, int nthreads, int grid, size_t lds, hipStream_t s, const KArgs& a) {
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3(grid), dim3(nthreads), lds, s, a);
  return hipGetLastError();
}

template <int QK, int MB, int WT, int KL>
hipError_t launch_one(const KArgs& a, int mode, int grid, size_t lds, hipStream_t s) {
  if (mode == kModeDense)
    return launch_kernel(dense_kernel<QK, MB, WT, KL, false>, kDenseWaves * 64, grid, lds, s, a);
  if (mode == kModeDenseGlobal)
    return launch_kernel(dense_kernel<QK, MB, WT, KL, true>, kDenseWaves * 64, grid, lds, s, a);
  if (a.rows_per_item == kStreamWavesLarge)
    return launch_kernel(stream_kernel<QK, MB, WT, KL, kStreamWavesLarge>, kStreamWavesLarge * 64,
                         grid, lds, s, a);
  if constexpr (QK == DT_FP8)
    return launch_kernel(stream_kernel<QK, MB, WT, KL, kStreamWaves>, kStreamWaves * 64, grid, lds,
                         s, a);
  else
    return launch_kernel(stream_shared_kernel<QK, MB, WT, KL>, kStreamWaves * 64, grid, lds, s, a);
}

template <int QK, int MB, int WT>
hipError_t launch_p(const KArgs& a, int mode, int kl, int grid, size_t lds, hipStream_t s) {
  switch (kl) {
    case KL_CONTIG: return launch_one<QK, MB, WT, KL_CONTIG>(a, mode, grid, lds, s);
    case KL_PAGED: return launch_one<QK, MB, WT, KL_PAGED>(a, mode, grid, lds, s);
    default: return launch_one<QK, MB, WT, KL_PAGED_TILE>(a, mode, grid, lds, s);
  }
}

template <int QK, int MB>
hipError_t launch_w(const KArgs& a, int mode, int w_dtype, int kl, int grid, size_t lds,
                    hipStream_t s) {
  return w_dtype == DT_FP32 ? launch_p<QK, MB, DT_FP32>(a, mode, kl, grid, lds, s)
                            : launch_p<QK, MB, DT_BF16>(a, mode, kl, grid, lds, s);
}

template <int QK>
hipError_t launch_mb(const KArgs& a, int mode, int w_dtype, int mblocks, int kl, int grid,
                     size_t lds, hipStream_t s) {
  return mblocks == 1 ? launch_w<QK, 1>(a, mode, w_dtype, kl, grid, lds, s)
                      : launch_w<QK, 2>(a, mode, w_dtype, kl, grid, lds, s);
}

}  // namespace

hipError_t launch_prefill(const KArgs& a, int mode, int qk_dtype, int w_dtype, int mblocks,
                          int kl, int grid, size_t lds, hipStream_t s) {
  switch (qk_dtype) {
    case DT_BF16: return launch_mb<DT_BF16>(a, mode, w_dtype, mblocks, kl, grid, lds, s);
    case DT_FP16: return launch_mb<DT_FP16>(a, mode, w_dtype, mblocks, kl, grid, lds, s);
    case DT_FP8: return launch_mb<DT_FP8>(a, mode, w_dtype, mblocks, kl, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace li
