// Exact k-th element selection for the top-k step.
//
// Order: value descending, then key index ascending (the smaller index wins a
// tie).  Given the k-th element (fb, eb) of that order, key e with value f is in
// the top k iff  f > fb  or  (f == fb and e <= eb).
//
// Method (bucket select, exact):
//   1. one histogram over 256 buckets linear in value between the candidates'
//      min and max (computed in fp32; the bucket map is monotone, so every key of
//      a higher bucket is strictly larger than every key of a lower bucket);
//   2. the bucket holding the k-th element is found from the suffix counts;
//   3. if it holds few candidates (<= 64) they are gathered and ranked exactly;
//      otherwise the search continues on that bucket with buckets of the
//      order-preserving u32 keys, each pass cutting the key range by 256, until
//      few candidates remain or all remaining candidates are equal, in which case
//      the tie rule alone decides (the r-th of them in index order).
// Values are never NaN; -0 has been folded into +0 by the producer.
#pragma once

#include <type_traits>

#include "li_device.h"

namespace li {

constexpr int kSelSmall = 64;

__device__ inline float wave_min_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline float wave_max_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ inline uint32_t wave_min_u(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = min(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}
__device__ inline uint32_t wave_max_u(uint32_t v) {
  for (int o = 32; o > 0; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  return v;
}

typedef LinBucket<256> FBucket;      // linear value buckets of the select
typedef KeyBucket<256> UBucket;      // u32 key buckets of its refining passes

// Finds, from 256 bucket counts (lane l owns buckets 4l..4l+3), the bucket that
// holds the element of rank r (1-based) counted from the top.  Returns the
// bucket, the number of candidates in higher buckets and in the bucket itself.
__device__ inline void wave_find_bucket(const uint32_t* hist, int r, int& bkt, int& above, int& cnt) {
  const int l = lane_id();
  const uint32_t h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
  const int s = (int)(h0 + h1 + h2 + h3);
  const int suf = wave_suffix_sum(s);
  const int ab = suf - s;
  const bool mine = ab < r && r <= suf;
  int b = 0, a = 0, c = 0;
  if (mine) {
    if (ab + (int)h3 >= r) { b = 4 * l + 3; a = ab; c = h3; }
    else if (ab + (int)(h3 + h2) >= r) { b = 4 * l + 2; a = ab + h3; c = h2; }
    else if (ab + (int)(h3 + h2 + h1) >= r) { b = 4 * l + 1; a = ab + h3 + h2; c = h1; }
    else { b = 4 * l; a = ab + h3 + h2 + h1; c = h0; }
  }
  const uint64_t who = ballot(mine);
  const int src = who ? (int)__builtin_ctzll(who) : 0;
  bkt = __shfl(b, src);
  above = __shfl(a, src);
  cnt = __shfl(c, src);
}

// Exact rank of the (<= 64) gathered candidates, one per lane (lanes >= m idle):
// returns the element of rank r (1-based) in (value desc, index asc) order.
__device__ inline void wave_rank_small(float f, uint32_t e, int m, int r, float& fb, uint32_t& eb) {
  const int l = lane_id();
  int rank = 0;
  m = __builtin_amdgcn_readfirstlane(m);       // uniform: the loop broadcasts by readlane
  for (int j = 0; j < m; ++j) {
    const float fj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f), j));
    const uint32_t ej = (uint32_t)__builtin_amdgcn_readlane((int)e, j);
    rank += (fj > f || (fj == f && ej < e)) ? 1 : 0;
  }
  const bool hit = l < m && rank == r - 1;
  const uint64_t who = ballot(hit);
  const int src = who ? (int)__builtin_ctzll(who) : 0;
  fb = __shfl(f, src);
  eb = (uint32_t)__shfl((int)e, src);
}

constexpr int kRowUnroll = 16;

// f(p, valid, v) over vals[0, n) in index order, in batches of kRowUnroll
// rounds of 64 entries, lane l holding entry p = batch start + 64 u + l.  The
// batch's loads are issued together, and f is called for every round of the
// batch, with no branch around it, so that the rounds' work can interleave:
// lanes past n get valid = false (their load re-reads entry n - 1).  Calls are
// wave-uniform (f may ballot).
template <class F>
__device__ __forceinline__ void row_pass(const float* vals, int n, F f) {
  const int l = lane_id();
  for (int p0 = 0; p0 < n; p0 += 64 * kRowUnroll) {
    float v[kRowUnroll];
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int p = p0 + 64 * u + l;
      v[u] = vals[p < n ? p : n - 1];
    }
#pragma unroll
    for (int u = 0; u < kRowUnroll; ++u) {
      const int p = p0 + 64 * u + l;
      f(p, p < n, v[u]);
    }
  }
}

// Views of the entries a select runs over: pass(f) calls f(p, valid, v) for
// every entry p in order, lane by lane (wave-uniform calls, so f may ballot),
// with kRowUnroll loads in flight per lane; key(p) is entry p's key.
// ArrayView: one array (idx == nullptr: the key of entry p is p).
// MemUnionView: a row's running top-k, entries [0, n0), followed by its
// candidate list, entries n0 + [0, n1).  Either way keys ascend with p.
struct ArrayView {
  const float* v;
  const uint32_t* i;
  int n;
  __device__ uint32_t key(int p) const { return i ? i[p] : (uint32_t)p; }
  template <class F>
  __device__ __forceinline__ void pass(F f) const {
    row_pass(v, n, f);
  }
};
struct MemUnionView {
  const float* v0;
  const uint32_t* i0;
  int n0;
  const float* v1;
  const uint32_t* i1;
  int n1;
  __device__ uint32_t key(int p) const { return p < n0 ? i0[p] : i1[p - n0]; }
  template <class F>
  __device__ __forceinline__ void pass(F f) const {
    row_pass(v0, n0, f);
    row_pass(v1, n1, [&](int p, bool valid, float x) __attribute__((always_inline)) {
      f(n0 + p, valid, x);
    });
  }
};

// Gathers the (<= kSelSmall) candidates selected by `in(f)` into lane order
// via the wave's LDS scratch (2 kSelSmall floats + 2 kSelSmall u32; a lane
// with nothing to write stores to its own slot of the upper halves, so no
// branch splits the rounds), ascending position.  The pass records positions;
// the keys are read afterwards, all at once (a key in memory is a round trip).
template <class View, class Pred>
__device__ inline int wave_gather(const View& vw, float* sf, uint32_t* se, Pred in, float& cf,
                                  uint32_t& ce) {
  const int l = lane_id();
  int got = 0;
  vw.pass([&](int p, bool valid, float f) __attribute__((always_inline)) {
    const bool take = valid && in(f);
    const uint64_t m = ballot(take);
    const int slot = got + mbcnt(m);
    const int at = (take & (slot < kSelSmall)) ? slot : kSelSmall + l;
    sf[at] = f;
    se[at] = (uint32_t)p;
    got += __popcll(m);
  });
  wave_sync();
  cf = l < got ? sf[l] : 0.0f;
  const int pos = l < got ? (int)se[l] : 0;
  ce = l < got ? vw.key(pos) : 0u;
  wave_sync();
  return got;
}

// Wave-level k-th element of the view's entries [0, n): keys ascend with the
// position (a dense row, a list in key order, or two such ranges in order).
// lo / hi: bounds of the n values (lo <= every value <= hi; the min and max
// for speed).  hist: 256 + 64 u32 (a lane past the end counts into its own
// slot of the last 64, so no branch splits the rounds) and scr: 4 * kSelSmall
// words of LDS private to the wave.  1 <= k <= n.
template <class View>
__device__ inline void wave_kth_view(const View& vw, int n, int k, float lo, float hi,
                                     uint32_t* hist, uint32_t* scr, float& fb, uint32_t& eb) {
  const int l = lane_id();
  float* sf = reinterpret_cast<float*>(scr);
  uint32_t* se = scr + 2 * kSelSmall;
  int r = k;
  uint32_t ulo, uhi;
  // ---- pass 1: linear value buckets ------------------------------------
  if (lo < hi) {
    const FBucket fbk(lo, hi);
    for (int x = l; x < 256; x += 64) hist[x] = 0;
    wave_sync();
    vw.pass([&](int, bool valid, float f) __attribute__((always_inline)) {
      atomicAdd(&hist[valid ? fbk(f) : 256u + l], 1u);
    });
    wave_sync();
    int B, above, cnt;
    wave_find_bucket(hist, r, B, above, cnt);
    r -= above;
    wave_sync();
    const uint32_t ub = (uint32_t)B;
    if (cnt <= kSelSmall) {
      float cf;
      uint32_t ce;
      const int got = wave_gather(vw, sf, se, [&](float f) { return fbk(f) == ub; }, cf, ce);
      wave_rank_small(cf, ce, got, r, fb, eb);
      return;
    }
    // key range of the chosen bucket, then continue on u32 keys
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    vw.pass([&](int, bool valid, float f) __attribute__((always_inline)) {
      const bool in = valid && fbk(f) == ub;
      const uint32_t u = f2key(f);
      mn = in ? min(mn, u) : mn;
      mx = in ? max(mx, u) : mx;
    });
    ulo = wave_min_u(mn);
    uhi = wave_max_u(mx);
  } else {
    ulo = uhi = f2key(lo);
  }
  // ---- exact passes on u32 keys ------------------------------------------
  for (;;) {
    if (ulo == uhi) {
      // every remaining candidate equals this key: the r-th of them in key order
      fb = key2f(ulo);
      eb = 0;
      int seen = 0;
      vw.pass([&](int p, bool valid, float f) __attribute__((always_inline)) {
        const bool eq = valid && f2key(f) == ulo;
        const uint64_t m = ballot(eq);
        const int c = __popcll(m);
        if (seen < r && seen + c >= r) {           // uniform: the round that holds it
          const bool hit = eq && seen + mbcnt(m) == r - 1;
          const uint64_t who = ballot(hit);
          const int src = who ? (int)__builtin_ctzll(who) : 0;
          const uint32_t e = hit ? vw.key(p) : 0u;
          eb = (uint32_t)__shfl((int)e, src);
        }
        seen += c;
      });
      return;
    }
    const UBucket ubk(ulo, uhi);
    for (int x = l; x < 256; x += 64) hist[x] = 0;
    wave_sync();
    vw.pass([&](int, bool valid, float f) __attribute__((always_inline)) {
      const uint32_t u = f2key(f);
      const bool in = valid && u >= ulo && u <= uhi;
      atomicAdd(&hist[in ? ubk(u) : 256u + l], 1u);
    });
    wave_sync();
    int B, above, cnt;
    wave_find_bucket(hist, r, B, above, cnt);
    r -= above;
    wave_sync();
    const uint32_t nlo = ulo + ((uint32_t)B << ubk.shift);
    uint32_t nhi = (B == 255) ? uhi : nlo + ((1u << ubk.shift) - 1u);
    if (nhi > uhi) nhi = uhi;
    if (cnt <= kSelSmall && nlo != nhi) {
      float cf;
      uint32_t ce;
      const int got = wave_gather(vw, sf, se, [&](float f) {
        const uint32_t u = f2key(f);
        return u >= nlo && u <= nhi;
      }, cf, ce);
      wave_rank_small(cf, ce, got, r, fb, eb);
      return;
    }
    ulo = nlo;
    uhi = nhi;
  }
}

// wave_kth_view over one array: idx == nullptr means the key of entry p is p.
__device__ inline void wave_kth(const float* vals, const uint32_t* idx, int n, int k, float lo,
                                float hi, uint32_t* hist, uint32_t* scr, float& fb, uint32_t& eb) {
  wave_kth_view(ArrayView{vals, idx, n}, n, k, lo, hi, hist, scr, fb, eb);
}

// ---------------------------------------------------------------------------
// Two-pass top-k of a dense score row (one wave per row), in LDS or in global
// memory.  Each pass keeps kRowUnroll loads in flight per lane (for a global
// row every load is an L2 round trip); one histogram of NB linear buckets
// usually leaves at most kSelSmall values in the bucket of the k-th element:
// kLdsBuckets for rows of up to 4096 keys in LDS, kWideBuckets for longer rows
// in global memory.
// ---------------------------------------------------------------------------
constexpr int kWideBuckets = 2048;
constexpr int kLdsBuckets = 512;

// wave_find_bucket over NB counts (lane l owns buckets NB/64 * l .. NB/64 * (l+1) - 1).
template <int NB>
__device__ inline void wave_find_bucket_n(const uint32_t* hist, int r, int& bkt, int& above,
                                          int& cnt) {
  constexpr int PER = NB / 64;
  const int l = lane_id();
  const uint32_t* h = hist + PER * l;
  int s = 0;
#pragma unroll
  for (int j = 0; j < PER; ++j) s += (int)h[j];
  const int suf = wave_suffix_sum(s);
  const int ab = suf - s;
  const bool mine = ab < r && r <= suf;
  int b = 0, a = 0, c = 0;
  if (mine) {
    int acc = ab;
    for (int j = PER - 1; j >= 0; --j) {
      const int hj = (int)h[j];
      if (acc + hj >= r) {
        b = PER * l + j;
        a = acc;
        c = hj;
        break;
      }
      acc += hj;
    }
  }
  const uint64_t who = ballot(mine);
  const int src = who ? (int)__builtin_ctzll(who) : 0;
  bkt = __shfl(b, src);
  above = __shfl(a, src);
  cnt = __shfl(c, src);
}

// Top-k of a dense score row vals[0, n) whose values lie in [lo, hi] (the
// index of entry p is p; k < n), written to oi / ov (indices plus ioff) in two
// passes: a histogram of NB buckets finds the bucket B of the k-th
// element; the second pass writes every entry of a bucket above B (all kept, in
// index order) and gathers bucket B, whose exact rank then decides which of its
// entries follow them.  Returns false, writing nothing, when lo == hi or bucket B
// holds more than kSelSmall entries.  hist: NB u32 and scr: 2 * kSelSmall
// words of LDS private to the wave.
template <int NB>
__device__ __forceinline__ bool wave_topk_row(const float* vals, int n, int k, float lo, float hi,
                                     uint32_t* hist, uint32_t* scr, int32_t* oi, float* ov,
                                     int ioff) {
  if (!(lo < hi)) return false;
  const int l = lane_id();
  const LinBucket<NB> fbk(lo, hi);
  for (int x = l; x < NB; x += 64) hist[x] = 0;
  wave_sync();
  row_pass(vals, n, [&](int, bool valid, float f) __attribute__((always_inline)) {
    if (valid) atomicAdd(&hist[fbk(f)], 1u);
  });
  wave_sync();
  int B, above, cnt;
  wave_find_bucket_n<NB>(hist, k, B, above, cnt);
  wave_sync();
  if (cnt > kSelSmall) return false;
  float* sf = reinterpret_cast<float*>(scr);
  uint32_t* se = scr + kSelSmall;
  int pos = 0, got = 0;
  // one predicated store region per entry (the values array's presence is a
  // compile-time branch); bucket B is rare, so its gathering sits behind a
  // uniform test of its ballot
  auto pass2 = [&](auto has_ov) __attribute__((always_inline)) {
    row_pass(vals, n, [&](int p, bool valid, float f) __attribute__((always_inline)) {
      const uint32_t bk = fbk(f);
      const bool up = valid & (bk > (uint32_t)B);
      const uint64_t mu = ballot(up);
      const int o = pos + mbcnt(mu);
      if (up & (o < k)) {
        oi[o] = p + ioff;
        if constexpr (decltype(has_ov)::value) ov[o] = f;
      }
      pos += __popcll(mu);
      const bool take = valid & (bk == (uint32_t)B);
      const uint64_t mt = ballot(take);
      if (mt != 0) {
        const int slot = got + mbcnt(mt);
        if (take & (slot < kSelSmall)) {
          sf[slot] = f;
          se[slot] = (uint32_t)p;
        }
        got += __popcll(mt);
      }
    });
  };
  if (ov) pass2(std::true_type{});
  else pass2(std::false_type{});
  wave_sync();
  const int m = got < kSelSmall ? got : kSelSmall;
  const float cf = l < m ? sf[l] : 0.0f;
  const uint32_t ce = l < m ? se[l] : 0u;
  wave_sync();
  float fb;
  uint32_t eb;
  wave_rank_small(cf, ce, m, k - above, fb, eb);
  // the gathered entries are in index order: the kept ones follow the others
  const bool keep = l < m && (cf > fb || (cf == fb && ce <= eb));
  const uint64_t mk = ballot(keep);
  const int o = above + mbcnt(mk);
  if (keep && o < k) {
    oi[o] = (int32_t)ce + ioff;
    if (ov) ov[o] = cf;
  }
  return true;
}

// The same, out of line: the score loop around it already holds most
// registers (rows in global memory), and a call keeps the select's registers
// out of that allocation.
template <int NB>
__device__ __noinline__ bool wave_topk_row_call(const float* vals, int n, int k, float lo, float hi,
                                                uint32_t* hist, uint32_t* scr, int32_t* oi,
                                                float* ov, int ioff) {
  return wave_topk_row<NB>(vals, n, k, lo, hi, hist, scr, oi, ov, ioff);
}

}  // namespace li
