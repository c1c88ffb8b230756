// Backward of the Lightning Indexer fused with its KL loss
// (npu_sparse_lightning_indexer_grad_kl_loss page, 计算公式 items 1-4).
//
// For query token t and its selected keys s_j (the valid entries of
// sparse_indices[t]):
//   I_j   = sum_h w_h ReLU(S_h,j),  S_h,j = qi[t,h] . ki[s_j]                    (item 1)
//   p_j   = sum_g exp(scale * (q[t,g] . k[s_j] + qr[t,g] . kr[s_j]) - max_g) / sum_g,
//           L1-normalised over j (the main attention's probabilities, recomputed
//           from the statistics its forward saved, summed over heads)             (item 2)
//   loss  = sum_t KL(p || Softmax(I))                                              (item 3)
//   dI    = Softmax(I) - p,  dW_h = sum_j dI_j ReLU(S_h,j),  dS = dI w [S > 0],
//   dqi   = dS @ ki[s],  dki[s] += dS^T @ qi                                       (item 4)
//
// One wave owns one query row (four independent rows per workgroup).  Its
// selected keys are gathered 32 at a time into the wave's LDS tiles; every
// contraction is an MFMA with the forward's fragment layout:
//   phase 1: S (heads x keys, as in the forward) and the main-attention logits
//            (main heads x keys, plus the rope part), then I and the head-summed
//            probabilities of each entry into LDS;
//   phase 2: softmax, the row's loss and dI, in LDS;
//   phase 3a: S^T (keys x heads) again, dW, and dqi += dS x ki with dS split
//            into bf16 (fp16) high and low parts, so that the product keeps fp32
//            accuracy;
//   phase 3b: S^T again, dS through LDS into the (keys x heads) operand, and
//            dki rows += dS x qi as one MFMA tile, added to the output with fp32
//            atomics (a key's gradient sums over every row that selected it).
#include "li_common_kernels.h"
#include "li_pipe.h"

namespace li {

namespace {

constexpr int kRopeRB = 128;       // bytes of a 64-dim rope row
constexpr int kLossThreads = 1024;

__device__ inline float wave_sum_f(float v) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  return v;
}
__device__ inline float wave_max_fv(float v) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

// Gathers the RB-byte rows of 32 keys into an LDS tile (16-byte chunk c of row r
// at chunk c ^ (r % (RB / 16)), the forward's swizzle).  key_lane: lane e < 32
// holds the key of tile row e (a token row of `src`).
template <int RB>
__device__ inline void gather_tile(unsigned char* tile, const void* src, int64_t key_lane,
                                   int lane) {
  constexpr int NCH = RB / 16, PER = 32 * NCH / 64;
  const unsigned char* base = reinterpret_cast<const unsigned char*>(src);
  i32x4 v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int id = lane + 64 * u, row = id / NCH, c = id % NCH;
    const int64_t key = __shfl(key_lane, row);
    v[u] = *reinterpret_cast<const i32x4*>(base + key * RB + c * 16);
  }
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int id = lane + 64 * u, row = id / NCH, c = id % NCH;
    *reinterpret_cast<i32x4*>(tile + row * RB + ((c ^ (row & (NCH - 1))) << 4)) = v[u];
  }
}

// 2-byte element (row, d) of a 256-byte-row tile in that swizzle
template <int QK>
__device__ inline uint16_t tile_elem(const unsigned char* tile, int row, int d) {
  return *reinterpret_cast<const uint16_t*>(tile + lds_chunk_off<QK>(row, d >> 3) + (d & 7) * 2);
}

// fp32 -> the 16-bit MFMA element type (round to nearest even), as raw bits
template <int QK>
__device__ inline uint16_t to_elem(float x) {
  if constexpr (QK == DT_FP16) {
    const _Float16 h = (_Float16)x;
    return __builtin_bit_cast(uint16_t, h);
  } else {
    const __bf16 h = (__bf16)x;
    return __builtin_bit_cast(uint16_t, h);
  }
}
template <int QK>
__device__ inline float from_elem(uint16_t u) {
  if constexpr (QK == DT_FP16) return (float)__builtin_bit_cast(_Float16, u);
  else return __uint_as_float((uint32_t)u << 16);
}

template <int QK>
__device__ inline typename Mma<QK>::frag pack8(const uint16_t (&e)[8]) {
  i32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (int)e[2 * i] | ((int)e[2 * i + 1] << 16);
  return __builtin_bit_cast(typename Mma<QK>::frag, v);
}

// Key of accumulator row r in the lane's half (the k-order the dq operands share).
__device__ inline int acc_key(int lane, int r) { return acc_row(lane, r); }

template <int QK, int WT, bool ROPE>
__global__ __launch_bounds__(kGradWaves * 64, 1) void grad_rows_kernel(GradArgs g) {
  typedef Mma<QK> M;
  typedef typename M::frag F;
  static_assert(M::RB == 256 && M::KSTEPS == 8, "16-bit q / k of 128 dims");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int64_t t = (int64_t)blockIdx.x * kGradWaves + wave;
  if (t >= g.rows) return;                       // the waves never synchronise with each other
  unsigned char* base = smem + (size_t)wave * (kGradTileBytes + 8 * (size_t)g.topk_pad);
  unsigned char* tileI = base;                   // index key rows (8 KiB)
  unsigned char* tileM = base + 8192;            // main key rows (8 KiB); phase 3b: dS^T
  unsigned char* tileR = base + 16384;           // rope key rows (4 KiB)
  float* arrI = reinterpret_cast<float*>(base + kGradTileBytes);   // I, then dI
  float* arrP = arrI + g.topk_pad;                                   // head-summed probabilities

  // batch of the row, its key offset and key count
  int64_t k_off;
  int s2;
  if (g.layout == L_TND) {
    int lo = 0, hi = g.batch - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (t < g.cu_q[mid]) hi = mid; else lo = mid + 1;
    }
    k_off = lo ? g.cu_k[lo - 1] : 0;
    s2 = (int)(g.cu_k[lo] - k_off);
  } else {
    const int b = (int)(t / g.s1);
    k_off = (int64_t)b * g.s2;
    s2 = g.s2;
  }
  const int32_t* sel = g.sel + t * g.topk;
  // entries past the last valid one are skipped tile-wise
  int last = -1;
  for (int j = lane; j < g.topk; j += 64) {
    const int e = sel[j];
    if (e >= 0 && e < s2) last = j;
  }
  for (int o = 32; o > 0; o >>= 1) last = max(last, __shfl_xor(last, o));
  const int ntiles = (last + 32) / 32;          // 0 when nothing is selected
  // the entry of tile row `lane` (lanes 0-31) and its key token (an invalid
  // entry reads key 0 of the batch: its results are masked)
  auto tile_key = [&](int j0, bool& ok) -> int64_t {
    const int j = j0 + (lane & 31);
    const int e = j < g.topk ? sel[j] : -1;
    ok = e >= 0 && e < s2;
    return k_off + (ok ? e : 0);
  };

  const int Ni = g.Ni, G = g.G;
  // ---- index query operands (A of S, B of S^T) and weights -------------------
  F qf[2][8];
  float wv[2][16];
  {
    KArgs ka;
    __builtin_memset(&ka, 0, sizeof(ka));
    ka.q = g.qi;
    ka.w = g.w;
    ka.n1 = Ni;
    load_query<QK, 2, WT>(ka, t, lane, qf, wv);
  }
  float row_loss = 0.0f;

  if (ntiles > 0) {
    // ---- phase 1: I and the head-summed main probabilities of each entry ------
    {
      F qm[2][8];
      F qr[2][4];
      float cb[2][16];                  // per head: (-max - ln sum) * log2(e); -inf past G
      const float l2e = 1.4426950408889634f;
      const float s2c = g.scale * l2e;
      const unsigned char* qrow = reinterpret_cast<const unsigned char*>(g.q) + t * G * 256;
      const unsigned char* rrow =
          ROPE ? reinterpret_cast<const unsigned char*>(g.q_rope) + t * G * kRopeRB : nullptr;
#pragma unroll
      for (int mb = 0; mb < 2; ++mb) {
        const int head = mb * 32 + (lane & 31);
        const bool in = head < G;
        const int hc = in ? head : 0;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          qm[mb][j] = load_frag_global<QK>(qrow + hc * 256 + frag_off<QK>(lane, j));
          if (!in) qm[mb][j] = zero_frag<QK>();
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if constexpr (ROPE) {
            qr[mb][j] = load_frag_global<QK>(rrow + hc * kRopeRB + (lane >> 5) * 64 + j * 16);
            if (!in) qr[mb][j] = zero_frag<QK>();
          } else {
            qr[mb][j] = zero_frag<QK>();
          }
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int h = mb * 32 + acc_row(lane, r);
          const int hh = h < G ? h : 0;
          const float c = -(g.smax[t * G + hh] + __logf(g.ssum[t * G + hh])) * l2e;
          cb[mb][r] = h < G ? c : -__builtin_inff();
        }
      }
      settle_loads();
      for (int tt = 0; tt < ntiles; ++tt) {
        const int j0 = tt * 32;
        bool ok;
        const int64_t key = tile_key(j0, ok);
        gather_tile<256>(tileI, g.ki, key, lane);
        gather_tile<256>(tileM, g.k, key, lane);
        if constexpr (ROPE) gather_tile<kRopeRB>(tileR, g.k_rope, key, lane);
        wave_sync();
        F kb[8];
        read_tile_frags<QK>(tileI, lane, kb);
        f32x16 accS[2];
        mma_tile<QK, 2>(qf, kb, accS);
        read_tile_frags<QK>(tileM, lane, kb);
        f32x16 accL[2];
        mma_tile<QK, 2>(qm, kb, accL);
        if constexpr (ROPE) {
          F kr[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int row = lane & 31, c0 = (lane >> 5) * 4 + j;
            const i32x4 v =
                *reinterpret_cast<const i32x4*>(tileR + row * kRopeRB + ((c0 ^ (row & 7)) << 4));
            kr[j] = __builtin_bit_cast(F, v);
          }
#pragma unroll
          for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int mb = 0; mb < 2; ++mb) accL[mb] = M::mma(qr[mb][j], kr[j], accL[mb]);
        }
        const float I = block_score<2>(accS, wv);
        float ps = 0.0f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            ps += __builtin_amdgcn_exp2f(fmaf(accL[mb][r], s2c, cb[mb][r]));
        ps = add_half_swap(ps);
        if (lane < 32) {
          arrI[j0 + lane] = ok ? I : -__builtin_inff();
          arrP[j0 + lane] = ok ? ps : 0.0f;
        }
        wave_sync();                            // the next gather overwrites the tiles
      }
    }

    // ---- phase 2: Softmax(I), the L1-normalised target, the loss and dI -------
    {
      const int n = ntiles * 32;
      float mx = -__builtin_inff();
      for (int j = lane; j < n; j += 64) mx = fmaxf(mx, arrI[j]);
      mx = wave_max_fv(mx);
      float se = 0.0f, z = 0.0f;
      for (int j = lane; j < n; j += 64) {
        se += __expf(arrI[j] - mx);
        z += arrP[j];
      }
      se = wave_sum_f(se);
      z = wave_sum_f(z);
      const float lse = mx + __logf(se);
      const float inv_z = 1.0f / z;
      for (int j = lane; j < n; j += 64) {
        const int e = j < g.topk ? sel[j] : -1;
        const bool ok = e >= 0 && e < s2;
        const float lpi = arrI[j] - lse;
        const float p = arrP[j] * inv_z;
        if (ok && p > 0.0f) row_loss += p * (__logf(p) - lpi);
        arrI[j] = ok ? __expf(lpi) - p : 0.0f;
      }
      row_loss = wave_sum_f(row_loss);
      wave_sync();
    }

    // ---- phase 3a: dW and dqi -------------------------------------------------
    {
      float wc[2];                              // the weight of this lane's head column
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int h = nb * 32 + (lane & 31);
        wc[nb] = h < Ni ? load_w<WT>(g.w, t * Ni + (h < Ni ? h : 0)) : 0.0f;
      }
      f32x16 dq[2][4];
      float dwp[2] = {0.0f, 0.0f};
#pragma unroll
      for (int nb = 0; nb < 2; ++nb)
#pragma unroll
        for (int db = 0; db < 4; ++db) dq[nb][db] = f32x16{};
      for (int tt = 0; tt < ntiles; ++tt) {
        const int j0 = tt * 32;
        bool ok;
        const int64_t key = tile_key(j0, ok);
        gather_tile<256>(tileI, g.ki, key, lane);
        wave_sync();
        F kb[8];
        read_tile_frags<QK>(tileI, lane, kb);
        // B operands of dqi: ki[key][d], keys in the accumulator's row order
        F bk[4][2];
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            uint16_t e[8];
            const int d = db * 32 + (lane & 31);
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) e[jj] = tile_elem<QK>(tileI, acc_key(lane, 8 * ks + jj), d);
            bk[db][ks] = pack8<QK>(e);
          }
        float dI[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 v = *reinterpret_cast<const float4*>(arrI + j0 + 8 * g4 + 4 * (lane >> 5));
          dI[4 * g4] = v.x;
          dI[4 * g4 + 1] = v.y;
          dI[4 * g4 + 2] = v.z;
          dI[4 * g4 + 3] = v.w;
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          f32x16 T = f32x16{};
#pragma unroll
          for (int j = 0; j < 8; ++j) T = M::mma(kb[j], qf[nb][j], T);   // S^T: keys x heads
          float ds[16];
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float x = T[r];
            dwp[nb] = fmaf(dI[r], relu(x), dwp[nb]);
            ds[r] = x > 0.0f ? dI[r] * wc[nb] : 0.0f;
          }
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            uint16_t hi[8], lo[8];
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const float v = ds[8 * ks + jj];
              hi[jj] = to_elem<QK>(v);
              lo[jj] = to_elem<QK>(v - from_elem<QK>(hi[jj]));
            }
            const F ah = pack8<QK>(hi), al = pack8<QK>(lo);
#pragma unroll
            for (int db = 0; db < 4; ++db) {
              dq[nb][db] = M::mma(ah, bk[db][ks], dq[nb][db]);
              dq[nb][db] = M::mma(al, bk[db][ks], dq[nb][db]);
            }
          }
        }
        wave_sync();
      }
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
#pragma unroll
        for (int db = 0; db < 4; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int h = nb * 32 + acc_row(lane, r);
            if (h < Ni) g.d_qi[(t * Ni + h) * 128 + db * 32 + (lane & 31)] = dq[nb][db][r];
          }
        const float v = dwp[nb] + __shfl_xor(dwp[nb], 32);
        const int h = nb * 32 + lane;
        if (lane < 32 && h < Ni) g.d_w[t * Ni + h] = v;
      }
    }

    // ---- phase 3b: dki -----------------------------------------------------------
    {
      // B operands of dki: qi[head][d], lane's column d, heads 16 ks + 8 half + jj
      const uint16_t* qrow = reinterpret_cast<const uint16_t*>(g.qi) + t * Ni * 128;
      F bq[4][4];
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          uint16_t e[8];
          const int d = db * 32 + (lane & 31);
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const int h = 16 * ks + 8 * (lane >> 5) + jj;
            e[jj] = h < Ni ? qrow[h * 128 + d] : (uint16_t)0;
          }
          bq[db][ks] = pack8<QK>(e);
        }
      float wc[2];
#pragma unroll
      for (int nb = 0; nb < 2; ++nb) {
        const int h = nb * 32 + (lane & 31);
        wc[nb] = h < Ni ? load_w<WT>(g.w, t * Ni + (h < Ni ? h : 0)) : 0.0f;
      }
      uint16_t* hiT = reinterpret_cast<uint16_t*>(tileM);          // [32 keys][64 heads]
      uint16_t* loT = hiT + 32 * 64;
      for (int tt = 0; tt < ntiles; ++tt) {
        const int j0 = tt * 32;
        bool ok;
        const int64_t key = tile_key(j0, ok);
        gather_tile<256>(tileI, g.ki, key, lane);
        wave_sync();
        F kb[8];
        read_tile_frags<QK>(tileI, lane, kb);
        float dI[16];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const float4 v = *reinterpret_cast<const float4*>(arrI + j0 + 8 * g4 + 4 * (lane >> 5));
          dI[4 * g4] = v.x;
          dI[4 * g4 + 1] = v.y;
          dI[4 * g4 + 2] = v.z;
          dI[4 * g4 + 3] = v.w;
        }
#pragma unroll
        for (int nb = 0; nb < 2; ++nb) {
          f32x16 T = f32x16{};
#pragma unroll
          for (int j = 0; j < 8; ++j) T = M::mma(kb[j], qf[nb][j], T);
          const int h = nb * 32 + (lane & 31);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float v = T[r] > 0.0f ? dI[r] * wc[nb] : 0.0f;
            const uint16_t hb = to_elem<QK>(v);
            hiT[acc_row(lane, r) * 64 + h] = hb;
            loT[acc_row(lane, r) * 64 + h] = to_elem<QK>(v - from_elem<QK>(hb));
          }
        }
        wave_sync();
        f32x16 dk[4];
#pragma unroll
        for (int db = 0; db < 4; ++db) dk[db] = f32x16{};
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int off = (lane & 31) * 64 + 16 * ks + 8 * (lane >> 5);
          const F ah = __builtin_bit_cast(F, *reinterpret_cast<const i32x4*>(hiT + off));
          const F al = __builtin_bit_cast(F, *reinterpret_cast<const i32x4*>(loT + off));
#pragma unroll
          for (int db = 0; db < 4; ++db) {
            dk[db] = M::mma(ah, bq[db][ks], dk[db]);
            dk[db] = M::mma(al, bq[db][ks], dk[db]);
          }
        }
        // rows of the tile: key of tile row acc_row(lane, r)
        const int64_t key_lane = ok ? key : -1;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t kr = __shfl(key_lane, acc_row(lane, r));
          if (kr >= 0) {
#pragma unroll
            for (int db = 0; db < 4; ++db)
              unsafeAtomicAdd(g.d_ki + kr * 128 + db * 32 + (lane & 31), dk[db][r]);
          }
        }
        wave_sync();                            // the next tile rewrites dS^T
      }
    }
  } else {
    // nothing selected: zero gradients for the row
    for (int e = lane; e < Ni * 128; e += 64) g.d_qi[t * Ni * 128 + e] = 0.0f;
    for (int e = lane; e < Ni; e += 64) g.d_w[t * Ni + e] = 0.0f;
  }
  if (lane == 0) g.loss_rows[t] = row_loss;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* p, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += step) p[e] = 0.0f;
}

// loss = sum of the rows' losses, in one fixed order (fp64 partial sums per
// thread over a fixed stride, then a fixed tree)
__global__ __launch_bounds__(kLossThreads) void loss_sum_kernel(const float* rows_loss, int n,
                                                               float* out) {
  __shared__ double part[kLossThreads];
  double s = 0.0;
  for (int i = threadIdx.x; i < n; i += kLossThreads) s += (double)rows_loss[i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int w = kLossThreads / 2; w > 0; w >>= 1) {
    if ((int)threadIdx.x < w) part[threadIdx.x] += part[threadIdx.x + w];
    __syncthreads();
  }
  if (threadIdx.x == 0) out[0] = (float)part[0];
}

template <int QK, int WT, bool ROPE>
hipError_t launch_rows(const GradArgs& g, hipStream_t s) {
  const size_t lds = (size_t)kGradWaves * (kGradTileBytes + 8 * (size_t)g.topk_pad);
  auto fn = grad_rows_kernel<QK, WT, ROPE>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(fn),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(fn, dim3((g.rows + kGradWaves - 1) / kGradWaves), dim3(kGradWaves * 64), lds,
                     s, g);
  return hipGetLastError();
}

template <int QK>
hipError_t launch_rows_w(const GradArgs& g, int w_dtype, bool rope, hipStream_t s) {
  if (w_dtype == DT_FP32)
    return rope ? launch_rows<QK, DT_FP32, true>(g, s) : launch_rows<QK, DT_FP32, false>(g, s);
  return rope ? launch_rows<QK, DT_BF16, true>(g, s) : launch_rows<QK, DT_BF16, false>(g, s);
}

}  // namespace

hipError_t launch_grad(const GradArgs& g, int qk_dtype, int w_dtype, bool rope, hipStream_t s) {
  if (g.keys > 0) {
    const int64_t n = g.keys * 128;
    const int64_t blocks = (n + 255) / 256 < 4096 ? (n + 255) / 256 : 4096;
    hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, g.d_ki, n);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (g.rows > 0) {
    hipError_t e = qk_dtype == DT_FP16 ? launch_rows_w<DT_FP16>(g, w_dtype, rope, s)
                                       : launch_rows_w<DT_BF16>(g, w_dtype, rope, s);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(loss_sum_kernel, dim3(1), dim3(kLossThreads), 0, s, g.loss_rows, g.rows,
                     g.loss);
  return hipGetLastError();
}

}  // namespace li
