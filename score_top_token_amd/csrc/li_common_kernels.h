// Pieces shared by the score kernels: visible-key limits, key addressing,
// operand loading and the ReLU.
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

// Visible keys of local row i of batch b: the right-down causal prefix, or for
// compressed keys (cmp_ratio r > 1, lightning_indexer page, parameters and
// Example) the keys whose r original positions j*r .. j*r + r - 1 all lie at or
// before the row's original position i + S2*r + residual - S1.
__device__ inline int row_limit(const KArgs& a, int b, int i, int s1, int s2) {
  if (a.cmp_ratio <= 1 || a.mask_mode == 0) return visible_limit(a.mask_mode, i, s1, s2);
  const long long r = a.cmp_ratio;
  const long long upto = (long long)i + 1 + (long long)s2 * r + a.cmp_res[b] - s1;  // positions <= it
  if (upto < r) return 0;
  const long long n = upto / r;
  return n >= s2 ? s2 : (int)n;
}

// The metadata header holds the fingerprint of the problem li_metadata built it
// for (lightning_indexer page, Prototype: the metadata call serves the indexer
// call of the same problem).  A kernel compares it with its own before reading
// any item.
__device__ inline bool meta_matches(const KArgs& a) {
  const MetaHeader* h = reinterpret_cast<const MetaHeader*>(a.meta);
  return h->magic == kMetaMagic && h->fingerprint == a.fingerprint;
}

// Records the call's status in the workspace (workgroup 0) and, when the
// metadata belongs to another problem, writes -1 / -inf into every output slot
// (the grid shares the rows, whose count comes from the problem, not from the
// metadata).  Returns whether the metadata matches; the caller then returns.
__device__ inline bool check_meta(const KArgs& a) {
  const bool ok = meta_matches(a);
  if (blockIdx.x == 0 && threadIdx.x == 0 && a.status) a.status[0] = ok ? 0 : kStatusMetaMismatch;
  if (!ok) {
    const int64_t n = (int64_t)a.rows * a.topk;
    const int64_t step = (int64_t)gridDim.x * blockDim.x;
    for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += step) {
      a.out_idx[e] = -1;
      if (a.out_val) a.out_val[e] = -__builtin_inff();
    }
  }
  return ok;
}

// Offset added to the written indices of batch b (output_idx_offset), else 0.
__device__ inline int index_offset(const KArgs& a, int b) { return a.idx_off ? a.idx_off[b] : 0; }

// Batch record written by the metadata kernel: {q token offset, S1_b, k token offset, S2_b}.
__device__ inline int4 batch_rec(const KArgs& a, int b) {
  return reinterpret_cast<const int4*>(a.meta + a.off_batch)[b];
}

// The same record computed from the call's own length arguments (lightning_indexer
// page, Constraints: inclusive cu_seqlens for TND, seqused_k for the paged keys,
// the fixed dimensions otherwise).  The metadata kernel writes exactly this; a
// kernel that needs only the lengths can read them without waiting for the
// metadata.  S1_b and S2_b are held to [0, S1max] and [0, S2max], the bounds
// every buffer is sized from (lengths past them are outside the contract).
__device__ inline int4 batch_lengths(const KArgs& a, int b) {
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
  s1 = min(max(s1, 0), a.s1max);
  s2 = min(max(s2, 0), a.s2max);
  return int4{q_off, s1, k_off, s2};
}

// Logical key s of batch b -> (paged pool block, row).  Power-of-two block
// sizes use shifts.
__device__ inline void paged_slot(const KArgs& a, int b, int s, int& blk, int& r) {
  int lb;
  if (a.block_shift >= 0) {
    lb = s >> a.block_shift;
    r = s & (a.block_size - 1);
  } else {
    lb = s / a.block_size;
    r = s - lb * a.block_size;
  }
  blk = a.block_table[(int64_t)b * a.max_blocks_per_seq + lb];
}

// Address of the RB-byte row of logical key s of batch b.
template <int QK, bool PAGED>
__device__ inline const unsigned char* key_row(const KArgs& a, int b, int k_off, int s) {
  constexpr int RB = Mma<QK>::RB;
  const unsigned char* base = reinterpret_cast<const unsigned char*>(a.k);
  if constexpr (PAGED) {
    int blk, r;
    paged_slot(a, b, s, blk, r);
    return base + (int64_t)blk * a.k_block_stride_bytes + (int64_t)r * RB;
  } else {
    return base + ((int64_t)k_off + s) * RB;
  }
}

// Descale slot of key s (paged: [block, row] of the pool; else the key token).
template <bool PAGED>
__device__ inline int64_t key_slot(const KArgs& a, int b, int k_off, int s) {
  if constexpr (PAGED) {
    int blk, r;
    paged_slot(a, b, s, blk, r);
    return (int64_t)blk * a.block_size + r;
  } else {
    return (int64_t)k_off + s;
  }
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

// LDS bytes one wave needs to stage a 32-head block of its query row.
template <int QK>
constexpr int q_stage_bytes() { return 32 * Mma<QK>::RB; }

// Q fragments (MFMA A operand) and per-lane weights of one query row.  Heads at or
// above n1 get zero q and zero weight, so they add nothing.
// A fragment load has each lane read 16 bytes of a different head row, so one
// instruction touches 64 cache lines for 1 KiB.  With kStaged the wave instead
// reads each 32-head block with 1 KiB-contiguous loads, parks it in its own
// q_stage_bytes() of LDS at `stage` (the K tiles' XOR swizzle, so the fragment
// reads spread over the banks) and reads the fragments back from there.
// `mid()` runs in the staged path once the query's loads are issued and before
// they are waited for, so that loads it issues queue behind them.
struct NoMid {
  __device__ void operator()() const {}
};
template <int QK, int MB, int WT, bool kStaged = false, class Mid = NoMid>
__device__ inline void load_query(const KArgs& a, int64_t tok, int lane,
                                  typename Mma<QK>::frag (&qf)[MB][Mma<QK>::KSTEPS],
                                  float (&wv)[MB][16], unsigned char* stage = nullptr,
                                  Mid mid = Mid()) {
  typedef Mma<QK> M;
  const unsigned char* qrow = reinterpret_cast<const unsigned char*>(a.q) + tok * a.n1 * M::RB;
  if constexpr (kStaged) {
    constexpr int NCH = M::RB / 16;            // 16-byte chunks per head row
    constexpr int NLD = 32 * NCH / 64;         // chunks per lane per block: 8 (bf16), 4 (fp8)
    i32x4 v[MB][NLD];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < NLD; ++r) {
        const int id = r * 64 + lane, hl = id / NCH, c = id % NCH;
        const int head = mb * 32 + hl;
        const bool in = head < a.n1;
        v[mb][r] = *reinterpret_cast<const i32x4*>(qrow + (int64_t)(in ? head : a.n1 - 1) * M::RB + c * 16);
        if (!in) v[mb][r] = i32x4{0, 0, 0, 0};
      }
    mid();
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
      for (int r = 0; r < NLD; ++r) {
        const int id = r * 64 + lane;
        *reinterpret_cast<i32x4*>(stage + lds_chunk_off<QK>(id / NCH, id % NCH)) = v[mb][r];
      }
      wave_sync();
#pragma unroll
      for (int j = 0; j < M::KSTEPS; ++j) qf[mb][j] = load_frag_lds<QK>(stage, lane & 31, lane, j);
      wave_sync();                               // the next block's stores follow these reads
    }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int head = mb * 32 + (lane & 31);
#pragma unroll
      for (int j = 0; j < M::KSTEPS; ++j)
        qf[mb][j] = head < a.n1 ? load_frag_global<QK>(qrow + head * M::RB + frag_off<QK>(lane, j))
                                : zero_frag<QK>();
    }
  }
  const float qd = (QK == DT_FP8) ? a.q_descale[tok] : 1.0f;
  // Accumulator rows 4g .. 4g+3 of a lane are 4 consecutive heads h0 .. h0+3
  // (h0 a multiple of 4).  Every weight load is issued unconditionally from a
  // clamped index and zeroed past n1 afterwards, so no branch splits them and
  // one wait covers them all.  With n1 % 4 == 0 and an aligned w the four
  // heads come in one vector load.
  const bool vec = (a.n1 & 3) == 0 &&
                   ((uintptr_t)a.w & (WT == DT_FP32 ? 15 : 7)) == 0;   // uniform
  if (vec) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int h0 = mb * 32 + acc_row(lane, 4 * g);
        const bool in = h0 < a.n1;
        const int64_t idx = tok * a.n1 + (in ? h0 : a.n1 - 4);
        float v[4];
        if constexpr (WT == DT_FP32) {
          const float4 x = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(a.w) + idx);
          v[0] = x.x; v[1] = x.y; v[2] = x.z; v[3] = x.w;
        } else {
          const uint2 x = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint16_t*>(a.w) + idx);
          v[0] = __uint_as_float(x.x << 16);
          v[1] = __uint_as_float(x.x & 0xFFFF0000u);
          v[2] = __uint_as_float(x.y << 16);
          v[3] = __uint_as_float(x.y & 0xFFFF0000u);
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) wv[mb][4 * g + q] = in ? v[q] * qd : 0.0f;
      }
  } else {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int h = mb * 32 + acc_row(lane, r);
        const bool in = h < a.n1;
        const float v = load_w<WT>(a.w, tok * a.n1 + (in ? h : a.n1 - 1));
        wv[mb][r] = in ? v * qd : 0.0f;
      }
  }
}

// Waits for every outstanding vector-memory load (the query operands) before a
// score loop.  Otherwise the wait-count analysis merges the loop entry (their
// loads pending) with the back edge (loads done) and waits for them, and so for
// every load issued after them, in each iteration.  0x0F70 encodes vmcnt(0)
// with expcnt and lgkmcnt left at their maxima.
__device__ inline void settle_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// max(x, 0) on the bit pattern: a negative float is a negative int32, so the
// integer max yields +0; one VALU op with no NaN canonicalisation.
__device__ inline float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

template <int QK, int MB>
__device__ inline void zero_query(typename Mma<QK>::frag (&qf)[MB][Mma<QK>::KSTEPS],
                                  float (&wv)[MB][16]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int j = 0; j < Mma<QK>::KSTEPS; ++j) qf[mb][j] = zero_frag<QK>();
#pragma unroll
    for (int r = 0; r < 16; ++r) wv[mb][r] = 0.0f;
  }
}

}  // namespace li
