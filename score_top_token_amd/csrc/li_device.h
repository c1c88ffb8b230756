// Device helpers for the gfx950 Lightning Indexer kernels: MFMA operand types,
// the d-permutation shared by the Q (A) and K (B) operands and wave-level
// primitives (the fp32 -> ordered u32 key map lives in li_bucket.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "li_bucket.h"
#include "li_internal.h"

namespace li {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(8 * sizeof(int)))) int i32x8;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

// ---------------------------------------------------------------------------
// MFMA traits.  One score tile is a 32 (heads) x 32 (keys) fp32 block built
// from D = 128 in KSTEPS instructions.  Each lane supplies FB bytes per step:
// lane l feeds head / key row (l % 32), and its half h = l / 32 holds the
// contiguous bytes [h * RB/2 + j * FB, + FB) of that row at step j.  A and B
// use the same byte -> d assignment, so any fixed permutation of d inside the
// instruction leaves every dot product intact.
// ---------------------------------------------------------------------------
template <int QK> struct Mma;

template <> struct Mma<DT_BF16> {
  static constexpr int RB = 256;      // bytes per q head row / k row
  static constexpr int FB = 16;       // bytes per lane per step
  static constexpr int KSTEPS = 8;
  typedef bf16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<DT_FP16> {
  static constexpr int RB = 256;
  static constexpr int FB = 16;
  static constexpr int KSTEPS = 8;
  typedef f16x8 frag;
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

template <> struct Mma<DT_FP8> {
  static constexpr int RB = 128;
  static constexpr int FB = 32;
  static constexpr int KSTEPS = 2;
  typedef i32x8 frag;
  // e4m3 x e4m3 with unit block scales (E8M0 exponent 127 = 2^0).
  __device__ static inline f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
  }
};

// Byte offset, inside a row, of the fragment lane `lane` feeds at step j.
template <int QK>
__device__ inline int frag_off(int lane, int j) {
  return (lane >> 5) * (Mma<QK>::RB / 2) + j * Mma<QK>::FB;
}

// Loads FB bytes from global memory as one fragment.
template <int QK>
__device__ inline typename Mma<QK>::frag load_frag_global(const unsigned char* p) {
  typedef typename Mma<QK>::frag F;
  F f;
  if constexpr (Mma<QK>::FB == 16) {
    i32x4 v = *reinterpret_cast<const i32x4*>(p);
    f = __builtin_bit_cast(F, v);
  } else {
    i32x4 v0 = *reinterpret_cast<const i32x4*>(p);
    i32x4 v1 = *reinterpret_cast<const i32x4*>(p + 16);
    i32x8 v = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    f = __builtin_bit_cast(F, v);
  }
  return f;
}

template <int QK>
__device__ inline typename Mma<QK>::frag zero_frag() {
  typedef typename Mma<QK>::frag F;
  if constexpr (Mma<QK>::FB == 16) {
    i32x4 v = {0, 0, 0, 0};
    return __builtin_bit_cast(F, v);
  } else {
    i32x8 v = {0, 0, 0, 0, 0, 0, 0, 0};
    return __builtin_bit_cast(F, v);
  }
}

// ---------------------------------------------------------------------------
// K tiles in LDS: kTileKeys rows of RB bytes; the 16-byte chunk c of row r is
// stored at chunk position c ^ (r % NCH), NCH = RB / 16, so the 32 rows one
// fragment read touches fall in distinct banks.
// ---------------------------------------------------------------------------
template <int QK>
__device__ inline int lds_chunk_off(int row, int chunk) {
  constexpr int NCH = Mma<QK>::RB / 16;
  return row * Mma<QK>::RB + ((chunk ^ (row & (NCH - 1))) << 4);
}

template <int QK>
__device__ inline typename Mma<QK>::frag load_frag_lds(const unsigned char* tile, int row, int lane,
                                                      int j) {
  typedef typename Mma<QK>::frag F;
  const int c0 = frag_off<QK>(lane, j) >> 4;
  if constexpr (Mma<QK>::FB == 16) {
    i32x4 v = *reinterpret_cast<const i32x4*>(tile + lds_chunk_off<QK>(row, c0));
    return __builtin_bit_cast(F, v);
  } else {
    i32x4 v0 = *reinterpret_cast<const i32x4*>(tile + lds_chunk_off<QK>(row, c0));
    i32x4 v1 = *reinterpret_cast<const i32x4*>(tile + lds_chunk_off<QK>(row, c0 + 1));
    i32x8 v = {v0[0], v0[1], v0[2], v0[3], v1[0], v1[1], v1[2], v1[3]};
    return __builtin_bit_cast(F, v);
  }
}

// ---------------------------------------------------------------------------
// Accumulator layout of a 32x32 fp32 MFMA block: lane l holds column l % 32 and,
// in element r (0..15), row 8 * (r / 4) + 4 * (l / 32) + (r % 4).
// ---------------------------------------------------------------------------
__device__ inline int acc_row(int lane, int r) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// ---------------------------------------------------------------------------
// Wave helpers (wave64)
// ---------------------------------------------------------------------------
__device__ inline int lane_id() { return __lane_id(); }

__device__ inline uint64_t ballot(bool p) { return __ballot(p); }

// number of set bits of m in lanes below this one
__device__ inline int mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ inline int wave_sum(int v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// inclusive suffix sum over lanes: returns sum of v over lanes >= this lane
__device__ inline int wave_suffix_sum(int v) {
  const int l = lane_id();
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_down(v, o);
    if (l + o < 64) v += t;
  }
  return v;
}

// inclusive prefix sum over lanes
__device__ inline int wave_prefix_sum(int v) {
  const int l = lane_id();
  for (int o = 1; o < 64; o <<= 1) {
    int t = __shfl_up(v, o);
    if (l >= o) v += t;
  }
  return v;
}

// v + (v of the lane 32 apart): the two halves of the wave exchanged by one
// v_permlane32_swap (VALU) instead of a bpermute through the LDS.  Float addition
// is commutative, so both lanes of a pair get the same bits.
__device__ inline float add_half_swap(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ inline void wave_sync() { __builtin_amdgcn_wave_barrier(); __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront"); }

}  // namespace li
