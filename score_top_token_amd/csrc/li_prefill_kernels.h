// Prefill kernels (templates; li_prefill_<dtype>.hip instantiate them, one
// translation unit per key dtype): scores of a block of query rows against
// every visible key, fused with an exact top-k per row.
//
// Score (npu_lightning_indexer_pto page, formula under "功能说明"; lightning_indexer
// page, "Function" steps 1-3): I[t,s] = sum_h w[t,h] * ReLU(q[t,h,:] . k[s,:]).
// The Q.K^T tile is an MFMA contraction with heads on M and keys on N; ReLU, the
// weights and the head sum run on the fp32 accumulators in registers.  One wave
// owns one query row; the workgroup shares each 64-key K tile through LDS.
//
// Top-k (lightning_indexer page, step 3; -1 / -inf padding from its Constraints):
// one kernel, 4 waves (rows) per workgroup, in three row modes by row length
// (dense_item below): every score of a row in LDS (rows up to 4096 keys; two
// workgroups share a CU at <= 80 KiB of LDS, so one workgroup's MFMAs run while
// the other is in its epilogue, select or output phase), every score in a
// workspace row (rows up to kGlobalRowKeys keys), or a bounded candidate list
// per row with a running threshold (longer rows).  The select is exact (ties to
// smaller keys); the kept keys fill the output prefix in an order that depends
// on the row mode but not on the run.
#pragma once

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

// Running top-k of a row streamed in key order (rows too long for LDS): `n_o`
// entries in the output slots oi / oval (ascending key), the threshold a new
// key has to beat, whether it may equal it (before the first real merge there
// is no k-th element and every key enters) and the entries' value range.
struct TopkState {
  int n_o;
  float thr;
  int incl;
  float omin, omax;
};

// Merges the `nl` LDS candidates listF / listI (keys above every top-k key)
// into the running top-k: keys oi in the output slots, values oval in LDS or
// in memory.  While everything fits the list is appended; otherwise the exact
// k-th element of the union is selected, the top-k is compacted (an entry only
// moves down) and the list's kept entries follow it, and the threshold rises
// to that element (later keys are larger, so they have to beat it).  Every
// pass keeps kRowUnroll (the compaction kMergeUnroll) rounds of loads in flight.  Called only where the
// pipeline has drained.  The top-k's entries move between lanes through
// memory; the same wave wrote them, so a workgroup-scope fence (a wait for the
// stores) makes them visible; an agent-scope one would write back and
// invalidate the whole L2.
constexpr int kMergeUnroll = 32;

__device__ __forceinline__ TopkState merge_list(const float* listF, const uint32_t* listI, int nl,
                                                int32_t* oi, float* oval, TopkState st, int topk,
                                                uint32_t* hist, uint32_t* scr) {
  const int lane = lane_id();
  float lo_l = __builtin_inff(), hi_l = -__builtin_inff();
  row_pass(listF, nl, [&](int, bool valid, float f) __attribute__((always_inline)) {
    lo_l = valid ? fminf(lo_l, f) : lo_l;
    hi_l = valid ? fmaxf(hi_l, f) : hi_l;
  });
  lo_l = wave_min_f(lo_l);
  hi_l = wave_max_f(hi_l);
  __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
  if (st.n_o + nl <= topk) {
    const int n_o = st.n_o;
    row_pass(listF, nl, [&](int p, bool valid, float f) __attribute__((always_inline)) {
      const uint32_t e = listI[valid ? p : nl - 1];
      if (valid) {
        oi[n_o + p] = (int32_t)e;
        oval[n_o + p] = f;
      }
    });
    st.n_o += nl;
    st.omin = fminf(st.omin, lo_l);
    st.omax = fmaxf(st.omax, hi_l);
    return st;
  }
  float fb;
  uint32_t eb;
  const MemUnionView vw{oval, reinterpret_cast<const uint32_t*>(oi), st.n_o, listF, listI, nl};
  wave_kth_view(vw, st.n_o + nl, topk, fminf(st.omin, lo_l), fmaxf(st.omax, hi_l), hist, scr, fb,
                eb);
  int w = 0;
  float kmin = __builtin_inff();
  auto put = [&](bool keep, float f, uint32_t e) __attribute__((always_inline)) {
    const uint64_t m = ballot(keep);
    const int pos = w + mbcnt(m);
    if (keep & (pos < topk)) {
      oi[pos] = (int32_t)e;
      oval[pos] = f;
      kmin = fminf(kmin, f);
    }
    w += __popcll(m);
  };
  // compaction in rounds of kMergeUnroll * 64 entries (a top-k of up to 2048
  // in one), the round's loads in flight together: an entry moves to a
  // position at or below its own, so a store never reaches an entry of this
  // or a later round that is still unread
  for (int p0 = 0; p0 < st.n_o; p0 += 64 * kMergeUnroll) {
    float f[kMergeUnroll];
    uint32_t e[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int p = p0 + 64 * u + lane;
      const int q = p < st.n_o ? p : st.n_o - 1;
      f[u] = oval[q];
      e[u] = (uint32_t)oi[q];
    }
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      if (p0 + 64 * u >= st.n_o) break;            // uniform
      const bool valid = p0 + 64 * u + lane < st.n_o;
      put(valid && (f[u] > fb || (f[u] == fb && e[u] <= eb)), f[u], e[u]);
    }
  }
  row_pass(listF, nl, [&](int p, bool valid, float f) __attribute__((always_inline)) {
    const uint32_t e = listI[valid ? p : nl - 1];
    put(valid && (f > fb || (f == fb && e <= eb)), f, e);
  });
  st.n_o = w < topk ? w : topk;            // exactly topk for ordered scores
  st.thr = fb;
  st.incl = 0;
  st.omin = wave_min_f(kmin);
  st.omax = fmaxf(st.omax, hi_l);
  return st;
}

// ---------------------------------------------------------------------------
// dense kernel: 4 rows per workgroup (one per wave) sharing each K tile.  The
// row mode RM says where a row's scores go:
//  kRowsLds: rows of at most `dcap` keys keep every score in LDS (one grid
//    slot per item); rows with no more visible keys than k are copied out
//    directly, the others go through the exact two-pass select;
//  kRowsGlobal: rows of up to kGlobalRowKeys keys keep every score in a
//    workspace row (L2 / HBM), one per wave of a fixed grid of two workgroups
//    per CU walking the work list; the same select follows, from memory;
//  kRowsList: longer rows (the same fixed grid) stream their top-k: each wave
//    keeps the row's running top-k in the row's own output slots (ascending key
//    order) and a list of up to `cap` candidates in LDS, the keys scoring above
//    the running threshold (the k-th score of the top-k so far).  A full list
//    is merged: the exact k-th element of (top-k so far) + (list) is selected,
//    the top-k is compacted in place and the list's kept entries appended after
//    it (their keys are larger), and the threshold rises to it.  No score row
//    leaves the chip.  The merge is a wave-serial select over about k + cap
//    entries, so it pays off only where rows are many times longer than k.
// ---------------------------------------------------------------------------
template <int QK, int MB, int WT, int KL, int RM>
__device__ __forceinline__ void dense_item(const KArgs& a, int it, unsigned char* smem) {
  constexpr bool L = RM == kRowsList;
  constexpr bool G = RM == kRowsGlobal;
  typedef Mma<QK> M;
  typedef typename M::frag F;
  constexpr int NT = kDenseWaves * 64;
  constexpr int TILE = kPipeKeys * M::RB;
  // [0, R0a): two K tiles and (fp8) the descale slots.
  //  kRowsLds / kRowsGlobal: the per-wave select scratch overlaps them after the
  //    score loop; LDS rows follow from R0;
  //  kRowsList: the per-wave merge scratch (used between pipeline runs) follows,
  //    then one int flag per wave, then the candidate lists (scores of every
  //    wave, then keys of every wave).
  constexpr int DSC = 2 * TILE;                      // descale slots (fp8 only)
  constexpr int R0a = DSC + (QK == DT_FP8 ? kDscSlots * 32 * 4 : 0);
  constexpr int SCR = L ? kListScratch : (G ? kWideScratch : kDenseScratch);
  constexpr int R0 = L ? R0a + kDenseWaves * SCR + 16
                      : (R0a > kDenseWaves * SCR ? R0a : kDenseWaves * SCR);
  float* dsc_lds = reinterpret_cast<float*>(smem + DSC);

  // opaque per item: lane-derived offsets are recomputed in each item instead of
  // being hoisted out of the item loop and held through the score loop
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int topk = a.topk;
  const int cap = a.cap;
  float* row = L ? nullptr
                 : (G ? a.ws + ((int64_t)blockIdx.x * kDenseWaves + wave) * a.ws_row_stride
                      : reinterpret_cast<float*>(smem + R0) + wave * a.dcap);
  float* listF = L ? reinterpret_cast<float*>(smem + R0) + wave * cap : nullptr;
  uint32_t* listI = L ? reinterpret_cast<uint32_t*>(smem + R0) + kDenseWaves * cap + wave * cap
                      : nullptr;
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
  // L: the values of the running top-k, in the output or (values not
  // requested) in the wave's workspace slot
  float* oval = ov ? ov : (L ? a.ws + ((int64_t)blockIdx.x * kDenseWaves + wave) * topk : nullptr);

  // fp8 tiles are half the registers: four in flight hide more of the L2 / MALL latency
  constexpr int D = QK == DT_FP8 ? 4 : kStageDepth;
  PipeStage<QK, KL, NT, D, RM != kRowsLds> st;
  st.prefetch_table(a, b, 0);
  F qf[MB][M::KSTEPS];                     // the query, loaded at the start of each run
  float wv[MB][16];

  // kRowsLds / kRowsGlobal: results of tile t (descaled) go to the row: lanes
  // 0-31 carry keys t*32 + lane, lanes 32-63 the same scores again.  Every
  // row's scores go to its row (the rows that need no select are copied out
  // after the loop), so a step's memory operations never depend on the row: a
  // data-dependent global store inside the loop would make every wait for the
  // K ring wait for it as well.  The row's minimum and maximum are tracked here.
  // kRowsList: keys above the threshold enter the wave's list (key order); until
  // the first real merge there is no k-th element and every key enters.
  float vmin = __builtin_inff(), vmax = -__builtin_inff();
  int n_l = 0;                             // list entries (uniform)
  TopkState ts{0, -__builtin_inff(), 1, __builtin_inff(), -__builtin_inff()};
  float thr = ts.thr;                      // wave-uniform copies read by the emit
  bool incl = true;
  auto emit = [&](int t, float tot) {
    const int s = t * kPipeKeys + (lane & 31);
    const bool in = lane < 32 && s < lim;
    if constexpr (L) {
      // threshold and the strictness of the comparison as one uniform test:
      // before the first real merge every key enters (f >= -inf), afterwards a
      // key has to beat the k-th score
      const float f = canon2(tot);
      const bool want = in & ((f > thr) | (incl & (f == thr)));
      const uint64_t m = ballot(want);
      if (m != 0) {                        // uniform
        const int pos = n_l + mbcnt(m);
        if (want & (pos < cap)) {          // always room; bounded whatever the data
          listF[pos] = f;
          listI[pos] = (uint32_t)(s + ioff);
        }
        n_l += __popcll(m);
      }
    } else if constexpr (G) {
      // every lane stores (lanes 32-63 repeat lanes 0-31); keys past lim land
      // below the row stride, in slots that are never read.  f is never NaN: a
      // compare and a select each, no operand quieting
      const float f = canon2(tot);
      row[s] = f;
      vmin = (in & (f < vmin)) ? f : vmin;
      vmax = (in & (f > vmax)) ? f : vmax;
    } else {
      // with rows in LDS the longer canonicalisation measures faster (schedule effect)
      const float f = canon(tot);
      if (in) row[s] = f;
      vmin = in ? fminf(vmin, f) : vmin;
      vmax = in ? fmaxf(vmax, f) : vmax;
    }
  };

  // L: the list into the running top-k (wave-level; merge_list)
  auto merge = [&]() __attribute__((always_inline)) {
    if constexpr (L) {
      const int nl = n_l < cap ? n_l : cap;
      if (nl == 0) return;
      uint32_t* hist = reinterpret_cast<uint32_t*>(smem + R0a + wave * kListScratch);
      ts = merge_list(listF, listI, nl, oi, oval, ts, topk, hist, hist + 320);
      thr = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(ts.thr)));
      incl = __builtin_amdgcn_readfirstlane(ts.incl) != 0;
      n_l = 0;
      wave_sync();                         // the list is refilled after this
    }
  };

  // L: one flag per wave, set when its list lacks room for another group of tiles
  int* need = L ? reinterpret_cast<int*>(smem + R0a + kDenseWaves * kListScratch) : nullptr;

  f32x16 accA[MB], accB[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    accA[mb] = f32x16{};
    accB[mb] = f32x16{};
  }
  float pend = 0.0f;                       // descaled scores of tile t-1, not yet emitted
  int t0 = 0;                              // first tile of the current pipeline run
  // Step t (ring set S = t % D): store tile t+1 into the other LDS buffer, load
  // tile t+D into set S, MFMAs of tile t into `cur` interleaved with the
  // epilogue of tile t-1 from `prev`, then tile t-2's scores are emitted: they
  // are a step old, so the emit never waits on the epilogue's latency.
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
    const float prev_score = block_score<MB, QK != DT_FP8>(prev, wv);
    // the per-key paged addressing leaves no room for every fragment at once
    pipe_schedule<QK, MB, KL != KL_PAGED>();
    __builtin_amdgcn_s_setprio(1);
    if (t > t0 + 1) emit(t - 2, pend);
    pend = QK == DT_FP8 ? prev_score * ds : prev_score;
    if constexpr (L && S == 3 % D) {
      // the last step of a group: is there room for another group and a drain?
      if (lane == 0) need[wave] = n_l > cap - kListRoom;
    }
    __syncthreads();
  };

  // One pipeline run from tile t0: full groups of 4 steps (two accumulator sets
  // x ring) run unconditionally, so every step issues the same loads and the
  // waits stay static counts; then the last 0-3 tiles, and the pipeline drains
  // with the last two emits.  L: a group adds at most 4 * 32 candidates and a
  // drain 2 * 32 (a tail with its final emits 5 * 32).  A run starts with at
  // least kListRoom = 6 * 32 free slots in every list; when a wave's list lacks
  // them after a group (the flags are set in the group's last step and read
  // after its barrier, so the decision is workgroup-uniform) the run stops
  // there and drains, the lists over half full are merged with nothing else
  // live, and a new run starts at the next tile.
  // Issue priority: a wave in its MFMA stretch first (2), then a wave in the
  // score loop (1), then a wave loading its query or selecting (0).  The SIMD's
  // other wave, from the other workgroup on the CU, is often in a different
  // phase; this keeps the matrix core fed from whichever wave has MFMAs ready.
  bool first = true;
  for (;;) {
    int t = t0;
    if (t0 < ntiles) {
      // The first run stages the query through LDS (coalesced loads; each wave's
      // staging area overlaps the K tiles, the rows and the lists, so all waves
      // finish with it first).  A later run (L) reads the fragments straight from
      // memory, the lists being in use: the query is then dead across the merges
      // between runs, which get the registers it holds.
      if (first) {
        if (has_row) load_query<QK, MB, WT, true>(a, tok, lane, qf, wv, smem + wave * q_stage_bytes<QK>());
        else zero_query<QK, MB>(qf, wv);
        settle_loads();
        __syncthreads();
      } else {
        if (has_row) load_query<QK, MB, WT, false>(a, tok, lane, qf, wv);
        else zero_query<QK, MB>(qf, wv);
      }
      first = false;
      st.template load<0>(a, b, br.z, t0 * kPipeKeys, kend, tid);
      st.template load<1>(a, b, br.z, (t0 + 1) * kPipeKeys, kend, tid);
      if constexpr (D > 2) {
        st.template load<2 % D>(a, b, br.z, (t0 + 2) * kPipeKeys, kend, tid);
        st.template load<3 % D>(a, b, br.z, (t0 + 3) * kPipeKeys, kend, tid);
      }
      st.template store<0>(smem + (t0 & 1) * TILE, tid);
      st.template store_dsc<0>(dsc_lds + (t0 & (kDscSlots - 1)) * 32, tid);
      __syncthreads();
      bool go = true;
      __builtin_amdgcn_s_setprio(1);
      while (go && t + 4 <= ntiles) {
        step(IntC<0>(), t, accA, accB);
        step(IntC<1>(), t + 1, accB, accA);
        step(IntC<2 % D>(), t + 2, accA, accB);
        step(IntC<3 % D>(), t + 3, accB, accA);
        t += 4;
        if constexpr (L) go = (need[0] | need[1] | need[2] | need[3]) == 0;
      }
      if (go) {
        if (t < ntiles) step(IntC<0>(), t, accA, accB);
        if (t + 1 < ntiles) step(IntC<1>(), t + 1, accB, accA);
        if (t + 2 < ntiles) step(IntC<2 % D>(), t + 2, accA, accB);
        t = ntiles;
      }
      const int last = t - 1;              // the run covered tiles t0 .. last
      const float ds = QK == DT_FP8 ? dsc_lds[(last & (kDscSlots - 1)) * 32 + (lane & 31)] : 1.0f;
      constexpr bool kSwap = QK != DT_FP8;
      const float sc = (last & 1) ? block_score<MB, kSwap>(accB, wv) : block_score<MB, kSwap>(accA, wv);
      if (last > t0) emit(last - 1, pend);
      emit(last, QK == DT_FP8 ? sc * ds : sc);
    }
    if constexpr (!L) {
      break;
    } else {
      // one merge site: between runs for every list over half full (the lists
      // that stopped the run among them; the waves merge side by side, so the
      // next stops come later), and at the end for every list, which leaves
      // exactly min(k, visible) entries in key order
      const bool fin = t >= ntiles;
      __builtin_amdgcn_s_setprio(0);
      if (fin || n_l > cap / 2) merge();
      if (fin) break;
      __syncthreads();                     // the next run restages tile t into LDS
      t0 = t;
    }
  }
  if constexpr (L) {
    if (has_row) write_padding(ts.n_o, topk, oi, ov);
    __syncthreads();                       // the next item stages its query over the lists
    return;
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
    // wide histogram, then the gather / rank scratch, then the bucket select's
    // own histogram
    uint32_t* hist = reinterpret_cast<uint32_t*>(smem + wave * kWideScratch);
    uint32_t* scr = hist + kWideBuckets;
    if (!wave_topk_row_call<kWideBuckets>(row, lim, topk, lo, hi, hist, scr, oi, ov, ioff)) {
      wave_kth(row, nullptr, lim, topk, lo, hi, scr + 4 * kSelSmall, scr, fb, eb);
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

template <int QK, int MB, int WT, int KL, int RM>
__global__ __launch_bounds__(kDenseWaves * 64, 2) void dense_kernel(KArgs a) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  if (!check_meta(a)) return;
  const int n_items = reinterpret_cast<const MetaHeader*>(a.meta)->n_items;
  if constexpr (RM == kRowsLds) {
    if ((int)blockIdx.x < n_items) dense_item<QK, MB, WT, KL, RM>(a, blockIdx.x, smem);
  } else {
    // The fixed grid walks the work list dynamically: a workgroup takes the
    // next item when it has finished one (a counter in the metadata header),
    // so the slots end together whatever the items' costs (a fixed stride
    // left the slots up to 10% apart).  The item number reaches every wave
    // through the first LDS word, between barriers: the LDS is free between
    // items (the select scratch and the lists are done with).
    MetaHeader* hdr = reinterpret_cast<MetaHeader*>(a.meta);
    int* s_item = reinterpret_cast<int*>(smem);
    for (;;) {
      __syncthreads();
      if (threadIdx.x == 0) s_item[0] = atomicAdd(&hdr->work_next, 1);
      __syncthreads();
      const int it = s_item[0];
      __syncthreads();                     // word 0 belongs to the item from here on
      if (it >= n_items) break;
      dense_item<QK, MB, WT, KL, RM>(a, it, smem);
    }
    // the last workgroup out leaves the counters at zero for the next call
    if (threadIdx.x == 0 && atomicAdd(&hdr->work_done, 1) == (int)gridDim.x - 1) {
      atomicExch(&hdr->work_next, 0);
      atomicExch(&hdr->work_done, 0);
    }
  }
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
    return launch_kernel(dense_kernel<QK, MB, WT, KL, kRowsLds>, kDenseWaves * 64, grid, lds, s, a);
  if (mode == kModeDenseGlobal)
    return launch_kernel(dense_kernel<QK, MB, WT, KL, kRowsGlobal>, kDenseWaves * 64, grid, lds, s, a);
  return launch_kernel(dense_kernel<QK, MB, WT, KL, kRowsList>, kDenseWaves * 64, grid, lds, s, a);
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

}  // namespace li
