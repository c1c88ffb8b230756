// Pieces shared by the score kernels: visible-key limits, key addressing,
// operand loading and the ReLU / weight / head-sum epilogue.
#pragma once

#include "li_device.h"

namespace li {

// Number of keys visible to local row i of a batch with s1 queries, s2 keys:
// mask 0 -> all keys; mask 3 (right-down causal) -> keys s <= i + s2 - s1.
__device__ inline int visible_limit(int mask_mode, int i, int s1, int s2) {
  if (mask_mode == 0) return s2;
  const long long last = (long long)i + s2 - s1;
  if (last < 0) return 0;
  return last >= s2 ? s2 : (int)(last + 1);
}

// Batch record written by the metadata kernel: {q token offset, S1_b, k token offset, S2_b}.
__device__ inline int4 batch_rec(const KArgs& a, int b) {
  return reinterpret_cast<const int4*>(a.meta + a.off_batch)[b];
}

// Address of the RB-byte row of logical key s of batch b, and its descale slot.
template <int QK>
__device__ inline const unsigned char* key_row(const KArgs& a, int b, int k_off, int s,
                                               int64_t* slot) {
  constexpr int ES = Mma<QK>::RB / kHeadDim;   // bytes per element
  const unsigned char* base = reinterpret_cast<const unsigned char*>(a.k);
  if (a.layout_k == L_PA) {
    const int lb = s / a.block_size;
    const int r = s - lb * a.block_size;
    const int blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + lb];
    if (slot) *slot = (int64_t)blk * a.block_size + r;
    return base + ((int64_t)blk * a.k_block_stride + (int64_t)r * kHeadDim) * ES;
  }
  const int64_t tok = (int64_t)k_off + s;
  if (slot) *slot = tok;
  return base + tok * Mma<QK>::RB;
}

template <int WT>
__device__ inline float load_w(const void* w, int64_t idx) {
  if constexpr (WT == DT_FP32) {
    return reinterpret_cast<const float*>(w)[idx];
  } else {
    const uint16_t u = reinterpret_cast<const uint16_t*>(w)[idx];
    return __uint_as_float(((uint32_t)u) << 16);
  }
}

// Q fragments (MFMA A operand) and per-lane weights of one query row.  Heads at or
// above n1 get zero q and zero weight, so they add nothing.
template <int QK, int MB, int WT>
__device__ inline void load_query(const KArgs& a, int64_t tok, int lane,
                                  typename Mma<QK>::frag (&qf)[MB][Mma<QK>::KSTEPS],
                                  float (&wv)[MB][16]) {
  typedef Mma<QK> M;
  const unsigned char* qrow = reinterpret_cast<const unsigned char*>(a.q) + tok * a.n1 * M::RB;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int head = mb * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < M::KSTEPS; ++j)
      qf[mb][j] = head < a.n1 ? load_frag_global<QK>(qrow + head * M::RB + frag_off<QK>(lane, j))
                              : zero_frag<QK>();
  }
  const float qd = (QK == DT_FP8) ? a.q_descale[tok] : 1.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int h = mb * 32 + acc_row(lane, r);
      wv[mb][r] = h < a.n1 ? load_w<WT>(a.w, tok * a.n1 + h) * qd : 0.0f;
    }
}

// ReLU, per-head weight and head sum of a 64-key tile held as acc[mb][nb]
// (nb = 32-key column block).  Returns, in lane l, the score of key l of the tile.
template <int MB>
__device__ inline float head_sum(const f32x16 (&acc)[MB][2], const float (&wv)[MB][16], int lane) {
  float p0 = 0.0f, p1 = 0.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p0 = fmaf(wv[mb][r], fmaxf(acc[mb][0][r], 0.0f), p0);
      p1 = fmaf(wv[mb][r], fmaxf(acc[mb][1][r], 0.0f), p1);
    }
  // lanes 0-31 hold half of the heads of keys 0-31 (p0) and 32-63 (p1); lanes
  // 32-63 the other half.  Exchange so lane l ends with the full sum of key l.
  const bool lo = lane < 32;
  const float send = lo ? p1 : p0;
  const float recv = __shfl_xor(send, 32);
  return (lo ? p0 : p1) + recv;
}

}  // namespace li
