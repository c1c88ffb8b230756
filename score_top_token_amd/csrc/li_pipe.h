// Software-pipelined score loop shared by the prefill kernels.
//
// The K stream is cut into 32-key tiles (one MFMA column block), double-buffered
// in LDS.  In iteration t a wave reads tile t's fragments, issues its MFMAs into
// one accumulator set and, interleaved with them, runs the ReLU / weight / head
// sum of tile t-1 from the other set, so the matrix cores and the vector ALUs
// work at the same time.  One barrier per tile: the store of tile t+1 into the
// other buffer and the loads of tile t+2 into registers overlap the compute.
#pragma once

#include <utility>

#include "li_common_kernels.h"

namespace li {

template <int N>
struct IntC {
  static constexpr int value = N;
};

// f(IntC<0>()), ..., f(IntC<N-1>()) in order
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(IntC<I>()), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>());
}

// fragments of one 32-key tile
template <int QK>
__device__ inline void read_tile_frags(const unsigned char* tile, int lane,
                                       typename Mma<QK>::frag (&kb)[Mma<QK>::KSTEPS]) {
#pragma unroll
  for (int j = 0; j < Mma<QK>::KSTEPS; ++j) kb[j] = load_frag_lds<QK>(tile, lane & 31, lane, j);
}

template <int QK, int MB>
__device__ inline void mma_tile(const typename Mma<QK>::frag (&qf)[MB][Mma<QK>::KSTEPS],
                                const typename Mma<QK>::frag (&kb)[Mma<QK>::KSTEPS],
                                f32x16 (&acc)[MB]) {
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x16{};
#pragma unroll
  for (int j = 0; j < Mma<QK>::KSTEPS; ++j)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) acc[mb] = Mma<QK>::mma(qf[mb][j], kb[j], acc[mb]);
}

// ReLU / weight / head sum of one 32-key block; lane l (and l + 32) ends with
// the score of key l % 32.  The two half-wave sums are joined by a VALU lane
// swap (kSwap) or by a bpermute through the LDS: the swap measures faster with
// 16-bit keys, the LDS exchange with fp8 keys, whose epilogue is bound by VALU
// issue.
template <int MB, bool kSwap = true>
__device__ inline float block_score(const f32x16 (&acc)[MB], const float (&wv)[MB][16]) {
  // one chain of fused multiply-adds: a wave64 VALU op takes four issue cycles,
  // which covers its latency, so the chain costs no more than split partial sums
  // and saves their final adds
  float s = 0.0f;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s = fmaf(wv[mb][r], relu(acc[mb][r]), s);
  if constexpr (kSwap) return add_half_swap(s);
  else return s + __shfl_xor(s, 32);
}

// Interleave hint for one pipelined iteration: each MFMA is followed by a few
// VALU instructions of the previous tile's epilogue.
template <int QK, int MB, bool kReadsFirst = true>
__device__ inline void pipe_schedule() {
  constexpr int NMFMA = MB * Mma<QK>::KSTEPS;
  constexpr int NVALU = MB * 32 + 8;
  constexpr int PER = (NVALU + NMFMA - 1) / NMFMA;
  constexpr int NREAD = Mma<QK>::KSTEPS * Mma<QK>::FB / 16;
  // every fragment read first (they queue in the LDS together, behind no MFMA),
  // then the MFMAs, each followed by VALU work of the epilogue; with
  // kReadsFirst = false the reads of the second half of the k-steps wait for the
  // first half's MFMAs, so half the fragment registers suffice
  constexpr int H = kReadsFirst ? 1 : 2;
#pragma unroll
  for (int h = 0; h < H; ++h) {
    __builtin_amdgcn_sched_group_barrier(0x100, NREAD / H, 0);
#pragma unroll
    for (int i = 0; i < NMFMA / H; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, PER, 0); // then VALU work
    }
  }
}

// Staging of 32-key K tiles by NT threads (global -> registers -> LDS) through
// a ring of D register sets, so a tile's loads are issued D steps before it is
// stored into LDS and the L2 latency hides behind D steps of compute.  In the
// tile that crosses kend the rows past it are re-read from row kend-1 (their
// scores are masked, their content is irrelevant).  A contiguous layout, or a paged one whose blocks hold a whole
// number of tiles (KL_PAGED_TILE), addresses a tile by one uniform base plus a
// constant 32-bit lane offset; other paged layouts look every key up.  Set
// indices are compile-time constants so the ring stays in registers.
// For fp8 keys the ring also carries the descale of the key that lane l % 32
// reports (dsc[S]), loaded right behind the tile so that waiting for it never
// drains the loads of later tiles; the workgroup kernels pass it on through an
// LDS slot per tile (kDscSlots slots of 32 floats).
// kClampOffset: a partial tile clamps the lanes' byte offsets (one min per
// load) rather than their keys (a min and a select per load).
template <int QK, int KL, int NT, int D, bool kClampOffset = false>
struct PipeStage {
  static constexpr int RB = Mma<QK>::RB;
  static constexpr int NCH = RB / 16;
  static constexpr int CHUNKS = kPipeKeys * NCH;
  static constexpr int LOADS = (CHUNKS + NT - 1) / NT;
  static_assert(CHUNKS % NT == 0, "a tile is an exact number of chunks per thread");
  static_assert(NT % NCH == 0, "a thread loads the same chunk column of each of its rows");
  i32x4 pre[D][LOADS];
  float dsc[D];
  // KL_PAGED_TILE: the physical ids of 64 consecutive logical blocks from
  // bt_first on, lane j of each wave holding block bt_first + j.  A tile's
  // block id is then a readlane, with no memory round trip in the step.
  int bt_lane = 0;
  int bt_first = -(1 << 30);

  __device__ inline void bt_fill(const KArgs& a, int b, int lb) {
    bt_first = lb;
    int j = lb + (int)(threadIdx.x & 63);
    j = j < a.max_blocks_per_seq ? j : a.max_blocks_per_seq - 1;
    bt_lane = a.block_table[(int64_t)b * a.max_blocks_per_seq + j];
  }
  // Issues the block-table load for the tiles from key `base` on (paged keys
  // only).  Called before the query loads, so that the first tile load waits
  // for this one load alone.
  __device__ inline void prefetch_table(const KArgs& a, int b, int base) {
    if constexpr (KL == KL_PAGED_TILE) bt_fill(a, b, logical_block(a, base));
  }
  __device__ static inline int logical_block(const KArgs& a, int s) {
    return a.block_shift >= 0 ? s >> a.block_shift : s / a.block_size;
  }

  // kend >= 1.  A tile at or past kend re-reads key kend-1 (cache hits), so
  // every call issues the same loads and the wait for a ring set is a static
  // count of the loads issued after it.
  template <int S>
  __device__ inline void load(const KArgs& a, int b, int k_off, int base, int kend, int tid) {
    base = base < kend ? base : kend - 1;            // uniform
    const int last = kend - 1 - base;                // last valid key of this tile
    const bool full = last >= kPipeKeys - 1;         // uniform
    if constexpr (KL == KL_PAGED) {
#pragma unroll
      for (int r = 0; r < LOADS; ++r) {
        const int id = tid + NT * r;
        int key = id / NCH;
        const int c = id % NCH;
        if (!full) key = key < last ? key : last;
        pre[S][r] = *reinterpret_cast<const i32x4*>(key_row<QK, true>(a, b, k_off, base + key) + c * 16);
      }
      if constexpr (QK == DT_FP8) {
        const int key = (tid & 31) < last ? (tid & 31) : last;
        dsc[S] = a.k_descale[key_slot<true>(a, b, k_off, base + key)];
      }
    } else {
      const unsigned char* tile;
      int64_t slot0;                                 // descale slot of the tile's first key
      if constexpr (KL == KL_PAGED_TILE) {
        const int lb = logical_block(a, base);
        const int r = base - lb * a.block_size;
        if ((unsigned)(lb - bt_first) >= 64u) {
          // past the 64 blocks held: reload (uniform, rare) and wait for it
          // here, so the readlane below never waits on the ring's loads
          bt_fill(a, b, lb);
          __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        const int blk = __builtin_amdgcn_readlane(bt_lane, lb - bt_first);
        tile = reinterpret_cast<const unsigned char*>(a.k) + (int64_t)blk * a.k_block_stride_bytes +
               (int64_t)r * RB;
        slot0 = (int64_t)blk * a.block_size + r;
      } else {
        tile = reinterpret_cast<const unsigned char*>(a.k) + ((int64_t)k_off + base) * RB;
        slot0 = (int64_t)k_off + base;
      }
      if constexpr (kClampOffset) {
        // byte offset of the lane's chunk, clamped to row `last`: the offset is
        // monotonic in the key, so clamping it clamps the key (a no-op for a
        // full tile); the bound is shared by the lane's loads (NT % NCH == 0)
        const uint32_t bound = (uint32_t)(last * RB + (tid % NCH) * 16);
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
          const int id = tid + NT * r;
          const uint32_t off = (uint32_t)((id / NCH) * RB + (id % NCH) * 16);
          pre[S][r] = *reinterpret_cast<const i32x4*>(tile + (off < bound ? off : bound));
        }
      } else {
#pragma unroll
        for (int r = 0; r < LOADS; ++r) {
          const int id = tid + NT * r;
          int key = id / NCH;
          const int c = id % NCH;
          if (!full) key = key < last ? key : last;
          pre[S][r] = *reinterpret_cast<const i32x4*>(tile + (uint32_t)(key * RB + c * 16));
        }
      }
      if constexpr (QK == DT_FP8) {
        const int key = (tid & 31) < last ? (tid & 31) : last;
        dsc[S] = a.k_descale[slot0 + key];
      }
    }
  }
  // fp8: the descales of the tile's 32 keys into an LDS slot (wave 0 writes)
  template <int S>
  __device__ inline void store_dsc(float* slot, int tid) const {
    if constexpr (QK == DT_FP8) {
      if (tid < 32) slot[tid] = dsc[S];
    }
  }
  template <int S>
  __device__ inline void store(unsigned char* tile, int tid) const {
#pragma unroll
    for (int r = 0; r < LOADS; ++r) {
      const int id = tid + NT * r;
      const int key = id / NCH, c = id % NCH;
      *reinterpret_cast<i32x4*>(tile + lds_chunk_off<QK>(key, c)) = pre[S][r];
    }
  }
};

// K ring depth (tiles in flight).  The dense kernel runs two workgroups per
// CU, whose register budget leaves room for 2 bf16 / fp16 tiles (it keeps 4 of
// the half-size fp8 tiles).
constexpr int kStageDepth = 2;
constexpr int kDscSlots = 4;      // tile t's descales live in slot t % 4 from step t-1 to t+1

}  // namespace li
