// Work-list builder (the lightning_indexer page's "lightning_indexer_metadata":
// a task list that tells each core which batch and which query / key block range
// to process, for load balancing).  One workgroup reads the per-batch lengths
// (inclusive cu_seqlens for TND, seqused_k for the paged layout, the fixed BSND
// dimensions otherwise) and writes
//   - a batch table {q token offset, S1_b, k token offset, S2_b},
//   - prefill modes: one item per block of `rows_per_item` query rows, ordered so
//     that the costliest blocks (the last rows of each sequence under right-down
//     causal masking) are dispatched first, round-robin over the batches with
//     the batch order rotated every round (workgroups are dealt to the 8 XCDs by
//     index mod 8: without the rotation a batch count that is a multiple of 8
//     would send every block of one batch to one XCD).  The dense kernel with
//     rows in global memory or in candidate lists walks the list with a stride
//     of its fixed grid, so there the list is batch-major instead (longest
//     sequence first, each from its last block): at any time every XCD works
//     on one sequence, whose keys then stay in its L2;
//   - decode mode: the visible keys of every query row cut into segments of one
//     length, the shortest for which all rows together need at most
//     kDecodeSegments segments; one item per segment.  The split kernel runs
//     kDecodeWaves items per workgroup, and workgroup w lands on XCD w mod 8,
//     whose share of HBM bandwidth bounds it: the full-length segments are dealt
//     round-robin over the XCDs, then the shorter last segments of the rows, and
//     the list is padded with empty items to whole rounds (batches up to
//     kRoundRobinMaxBatch; larger ones keep row order).
// The result depends only on the lengths (deterministic) and is produced on the
// device, so the call never synchronises with the host.
#include "li_pipe.h"
#include "li_select.h"

namespace li {

namespace {

constexpr int kMetaThreads = 1024;
constexpr int kRoundRobinMaxBatch = 256;
constexpr int kChunkCands = 8;      // decode: segment lengths tried at once

__device__ inline int cdiv(int a, int b) { return (a + b - 1) / b; }

// ceil(a / b) for 0 <= a < 2^53, b > 0: a double-precision quotient (hardware
// fp64 instead of a long emulated 64-bit integer division), corrected to the
// exact integer
__device__ inline long long cdiv64(long long a, long long b) {
  long long q = (long long)((double)a / (double)b);
  while (q * b < a) ++q;
  while (q > 0 && (q - 1) * b >= a) --q;
  return q;
}

// SMALL: batch <= kRoundRobinMaxBatch, the batch tables are also kept in LDS
template <bool SMALL>
__global__ __launch_bounds__(kMetaThreads) void metadata_kernel(KArgs a, int mode) {
  // small batches keep their tables in LDS as well: the later steps read them
  // from there instead of waiting on global memory round trips
  __shared__ int s_counts[kRoundRobinMaxBatch];
  __shared__ int s_starts[kRoundRobinMaxBatch];
  __shared__ int4 s_bt[kRoundRobinMaxBatch];
  __shared__ int s_part[kMetaThreads / 64];
  __shared__ int s_pstart[kRoundRobinMaxBatch];   // decode: partial segments before batch b
  __shared__ int s_npart;                          // decode: all partial segments
  __shared__ int s_gstart[kRoundRobinMaxBatch];    // batch-major prefill: first item of batch b
  __shared__ unsigned long long s_cand[kChunkCands], s_tot, s_nrows;
  __shared__ int s_total, s_chunk;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int B = a.batch;
  MetaHeader* hdr = reinterpret_cast<MetaHeader*>(a.meta);
  int4* bt = reinterpret_cast<int4*>(a.meta + a.off_batch);
  int* counts = reinterpret_cast<int*>(a.meta + a.off_counts);
  int* starts = reinterpret_cast<int*>(a.meta + a.off_starts);
  int4* items = reinterpret_cast<int4*>(a.meta + a.off_items);
  constexpr bool small = SMALL;
  auto get_bt = [&](int b) -> int4 {
    if constexpr (SMALL) return s_bt[b];
    else return bt[b];
  };
  auto get_count = [&](int b) -> int {
    if constexpr (SMALL) return s_counts[b];
    else return counts[b];
  };
  auto get_start = [&](int b) -> int {
    if constexpr (SMALL) return s_starts[b];
    else return starts[b];
  };

  // 1. per-batch lengths (and, for decode, the visible keys of its rows)
  long long vis = 0;
  for (int b = tid; b < B; b += kMetaThreads) {
    const int4 rec = batch_lengths(a, b);
    const int s1 = rec.y, s2 = rec.w;
    bt[b] = rec;
    if (small) s_bt[b] = rec;
    if (mode == kModeDecode)
      for (int i = 0; i < s1; ++i) vis += row_limit(a, b, i, s1, s2);
  }
  // decode segment length: the shortest multiple of 32 keys for which the
  // segments of all rows number at most `target` (one per wave of a full GPU,
  // kDecodeSegments, more if there are many rows).  Since every row adds at
  // most one partial segment, tot / (target - rows) always fits; the candidates
  // between tot / target and that bound are counted in one pass.
  if (SMALL && mode == kModeDecode) {
    // Small decode batches: wave 0 alone finds the segment length and the
    // per-batch counts, starts and short last segments (lane l holds batches
    // 4l .. 4l+3, so the scans run in batch order), with no block barrier in
    // between; the candidate lengths are counted with lane 8j + g taking
    // candidate j over every 8th batch from g.
    __syncthreads();                        // s_bt is complete
    if (wave == 0) {
      long long v = 0;
      int nr = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = 4 * lane + q;
        if (b < B) {
          const int4 rec = s_bt[b];
          nr += rec.y;
          for (int i = 0; i < rec.y; ++i) v += row_limit(a, b, i, rec.y, rec.w);
        }
      }
      for (int o = 32; o > 0; o >>= 1) {
        v += __shfl_xor(v, o);
        nr += __shfl_xor(nr, o);
      }
      const long long tot = v, nrows = nr;
      long long target = kDecodeSegments;
      while (target < 2 * nrows) target += kDecodeSegments;
      long long c_hi = (cdiv64(tot, target - nrows) + kPipeKeys - 1) / kPipeKeys * kPipeKeys;
      long long c_lo = (cdiv64(tot, target) + kPipeKeys - 1) / kPipeKeys * kPipeKeys;
      if (c_lo < a.chunk) c_lo = a.chunk;
      if (c_hi < c_lo) c_hi = c_lo;
      long long step = cdiv64(c_hi - c_lo, kChunkCands - 1);
      step = (step + kPipeKeys - 1) / kPipeKeys * kPipeKeys;
      if (step < kPipeKeys) step = kPipeKeys;
      static_assert(kChunkCands == 8, "eight candidates of eight lanes each");
      const int j = lane >> 3, g = lane & 7;
      const long long cj = j == kChunkCands - 1 ? c_hi : c_lo + j * step;
      const uint32_t c = (uint32_t)cj;
      unsigned long long ns = 0;
      for (int b = g; b < B; b += 8) {
        const int4 rec = s_bt[b];
        for (int i = 0; i < rec.y; ++i)
          ns += ((uint32_t)row_limit(a, b, i, rec.y, rec.w) + c - 1u) / c;
      }
      for (int o = 1; o < 8; o <<= 1) ns += __shfl_xor(ns, o);
      // the shortest candidate within the budget (c_hi always is)
      const bool ok = cj <= c_hi && (long long)ns <= target;
      const int chunk_w = (int)min(wave_min_u(ok ? c : 0xFFFFFFFFu), (uint32_t)c_hi);
      int cnt[4], pc[4], sc = 0, sp = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = 4 * lane + q;
        cnt[q] = pc[q] = 0;
        if (b < B) {
          const int4 rec = s_bt[b];
          for (int i = 0; i < rec.y; ++i) {
            const int lim = row_limit(a, b, i, rec.y, rec.w);
            cnt[q] += cdiv(lim, chunk_w);
            pc[q] += (lim % chunk_w) != 0;
          }
        }
        sc += cnt[q];
        sp += pc[q];
      }
      int run = wave_prefix_sum(sc) - sc, prun = wave_prefix_sum(sp) - sp;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int b = 4 * lane + q;
        if (b < B) {
          counts[b] = cnt[q];
          s_counts[b] = cnt[q];
          starts[b] = run;
          s_starts[b] = run;
          s_pstart[b] = prun;
        }
        run += cnt[q];
        prun += pc[q];
      }
      if (lane == 63) {
        s_total = run;
        s_npart = prun;
      }
      if (lane == 0) s_chunk = chunk_w;
    }
    __syncthreads();
  } else {
    if (mode == kModeDecode) {
      // block sums through LDS atomics (no serial loop over the waves)
      if (tid < kChunkCands) s_cand[tid] = 0;
      if (tid == 0) s_tot = s_nrows = 0;
      __syncthreads();
      long long rows = 0;
      for (int b = tid; b < B; b += kMetaThreads) rows += get_bt(b).y;
      for (int o = 32; o > 0; o >>= 1) {
        vis += __shfl_xor(vis, o);
        rows += __shfl_xor(rows, o);
      }
      if (lane == 0) {
        atomicAdd(&s_tot, (unsigned long long)vis);
        atomicAdd(&s_nrows, (unsigned long long)rows);
      }
      __syncthreads();
      const long long tot = (long long)s_tot, nrows = (long long)s_nrows;
      long long target = kDecodeSegments;
      while (target < 2 * nrows) target += kDecodeSegments;
      long long c_hi = (cdiv64(tot, target - nrows) + kPipeKeys - 1) / kPipeKeys * kPipeKeys;
      long long c_lo = (cdiv64(tot, target) + kPipeKeys - 1) / kPipeKeys * kPipeKeys;
      if (c_lo < a.chunk) c_lo = a.chunk;
      if (c_hi < c_lo) c_hi = c_lo;
      // candidate c_lo + j * step, j < kChunkCands; the last one is c_hi
      long long step = cdiv64(c_hi - c_lo, kChunkCands - 1);
      step = (step + kPipeKeys - 1) / kPipeKeys * kPipeKeys;
      if (step < kPipeKeys) step = kPipeKeys;
      // thread t counts candidate t % kChunkCands over every
      // (kMetaThreads / kChunkCands)-th batch; lanes of one candidate are then
      // summed with three shuffles and one LDS atomic per wave.  lim and c are
      // below 2^31: 32-bit unsigned division.
      {
        const int j = tid % kChunkCands;
        const uint32_t c = (uint32_t)(j == kChunkCands - 1 ? c_hi : c_lo + j * step);
        unsigned long long nseg = 0;
        for (int b = tid / kChunkCands; b < B; b += kMetaThreads / kChunkCands) {
          const int4 rec = get_bt(b);
          for (int i = 0; i < rec.y; ++i)
            nseg += ((uint32_t)row_limit(a, b, i, rec.y, rec.w) + c - 1u) / c;
        }
        for (int o = kChunkCands; o < 64; o <<= 1) nseg += __shfl_xor(nseg, o);
        if (lane < kChunkCands && nseg) atomicAdd(&s_cand[lane], nseg);
      }
      __syncthreads();
      if (tid == 0) {
        long long c = c_hi;
        for (int j = kChunkCands - 1; j >= 0; --j) {
          const long long cj = j == kChunkCands - 1 ? c_hi : c_lo + j * step;
          if (cj <= c_hi && (long long)s_cand[j] <= target && cj < c) c = cj;
        }
        s_chunk = (int)c;
      }
    } else if (tid == 0) {
      s_chunk = a.chunk;
    }
    __syncthreads();
    const int chunk = s_chunk;

    for (int b = tid; b < B; b += kMetaThreads) {
      const int4 rec = get_bt(b);
      int cnt = 0;
      if (mode == kModeDecode) {
        for (int i = 0; i < rec.y; ++i) cnt += cdiv(row_limit(a, b, i, rec.y, rec.w), chunk);
      } else {
        cnt = cdiv(rec.y, a.rows_per_item);
      }
      counts[b] = cnt;
      if (small) s_counts[b] = cnt;
    }
    __syncthreads();

    // 2. exclusive prefix of the counts (each thread scans a contiguous segment)
    const int seg = cdiv(B, kMetaThreads);
    const int b0 = tid * seg, b1 = min(b0 + seg, B);
    int local = 0;
    for (int b = b0; b < b1; ++b) local += get_count(b);
    const int incl = wave_prefix_sum(local);
    if (lane == 63) s_part[wave] = incl;
    __syncthreads();
    if (wave == 0) {                          // exclusive scan of the wave totals
      const int v = lane < kMetaThreads / 64 ? s_part[lane] : 0;
      const int inc = wave_prefix_sum(v);
      if (lane < kMetaThreads / 64) s_part[lane] = inc - v;
      if (lane == 63) s_total = inc;
    }
    __syncthreads();
    int run = s_part[wave] + incl - local;
    for (int b = b0; b < b1; ++b) {
      starts[b] = run;
      if (small) s_starts[b] = run;
      run += get_count(b);
    }
  }
  const int chunk = s_chunk;
  const int total = min(s_total, a.max_items);
  constexpr int kXcdRound = 8 * kDecodeWaves;
  const bool xcd_deal = small && mode == kModeDecode;
  int n_slots = total;
  if (xcd_deal) n_slots = min((total + kXcdRound - 1) / kXcdRound * kXcdRound, a.max_items);
  if (small && (mode == kModeDenseGlobal || mode == kModeDenseList)) {
    // batches by query rows, descending (ties by index): items before batch b
    for (int b = tid; b < B; b += kMetaThreads) {
      const int len = s_bt[b].y;
      int before = 0;
      for (int bb = 0; bb < B; ++bb) {
        const int l2 = s_bt[bb].y;
        before += (l2 > len || (l2 == len && bb < b)) ? s_counts[bb] : 0;
      }
      s_gstart[b] = before;
    }
  }
  if (tid == 0) {
    hdr->n_items = n_slots;
    hdr->mode = mode;
    hdr->chunk = chunk;
    hdr->magic = kMetaMagic;
    hdr->batch = B;
    hdr->max_items = a.max_items;
    hdr->fingerprint = a.fingerprint;
    hdr->work_next = 0;
    hdr->work_done = 0;
  }
  __syncthreads();

  // 3. items
  for (int u = tid; u < total; u += kMetaThreads) {
    // batch of the u-th item in batch-major order: last b with starts[b] <= u
    int lo = 0, hi = B - 1;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (get_start(mid) <= u) lo = mid; else hi = mid - 1;
    }
    const int b = lo;
    const int r = u - get_start(b);
    const int4 rec = get_bt(b);
    if (mode != kModeDecode) {
      const int cnt = get_count(b);
      const int blk = cnt - 1 - r;                 // r = 0 is the last (costliest) block
      const int q0 = blk * a.rows_per_item;
      const int nrows = min(a.rows_per_item, rec.y - q0);
      int pos = u;
      if (small && (mode == kModeDenseGlobal || mode == kModeDenseList)) {
        pos = s_gstart[b] + r;
      } else if (small) {
        // round-robin over batches, each batch walked from its last block.
        // Round r holds the n_r batches with more than r blocks; their order
        // is rotated by r, so that a batch does not land on the same XCD
        // (workgroup index mod 8) in every round:
        // pos = sum_b' min(r, cnt_b') + (#{b' < b : cnt_b' > r} + r) mod n_r
        int base = 0, idx = 0, nr = 0;
        for (int bb = 0; bb < B; ++bb) {
          const int c = s_counts[bb];
          base += min(r, c);
          idx += (bb < b && c > r) ? 1 : 0;
          nr += c > r ? 1 : 0;
        }
        pos = base + (idx + r) % nr;
      }
      if (pos < a.max_items) items[pos] = int4{b, q0, nrows, 0};
    } else {
      int rest = r, i = 0, lim = 0, part = 0;
      for (; i < rec.y; ++i) {
        lim = row_limit(a, b, i, rec.y, rec.w);
        const int nch = cdiv(lim, chunk);
        if (rest < nch) break;
        rest -= nch;
        part += (lim % chunk) != 0;
      }
      const int k0 = rest * chunk;
      const int k1 = min(k0 + chunk, lim);
      int pos = u;
      if (xcd_deal) {
        // rank j among the full segments (row order), or after all of them
        // among the partial ones; the j-th goes to XCD j mod 8
        const int pbefore = s_pstart[b] + part;
        const int j = k1 - k0 == chunk ? u - pbefore : total - s_npart + pbefore;
        const int k = j >> 3;
        pos = ((k / kDecodeWaves) * 8 + (j & 7)) * kDecodeWaves + k % kDecodeWaves;
      }
      if (pos < a.max_items) items[pos] = int4{b, i, k0, k1};
    }
  }
  // empty items in the slots no segment was dealt to
  if (xcd_deal) {
    for (int s = tid; s < n_slots; s += kMetaThreads) {
      const int k = (s / kDecodeWaves / 8) * kDecodeWaves + s % kDecodeWaves;
      const int j = k * 8 + (s / kDecodeWaves) % 8;
      if (j >= total) items[s] = int4{0, 0, 0, 0};
    }
  }
}

}  // namespace

hipError_t launch_metadata(const KArgs& a, int mode, hipStream_t s) {
  if (a.batch <= kRoundRobinMaxBatch)
    hipLaunchKernelGGL(metadata_kernel<true>, dim3(1), dim3(kMetaThreads), 0, s, a, mode);
  else
    hipLaunchKernelGGL(metadata_kernel<false>, dim3(1), dim3(kMetaThreads), 0, s, a, mode);
  return hipGetLastError();
}

}  // namespace li
