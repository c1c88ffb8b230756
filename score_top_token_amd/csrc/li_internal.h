// Internal definitions shared by the host dispatch (li_host.cpp) and the HIP
// kernels: the launch plan, the metadata layout and the kernel argument block.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace li {

constexpr int kHeadDim = 128;
constexpr int kMaxHeads = 64;
constexpr int kMaxTopk = 2048;         // any topk up to here; above it 3072 .. 8192 in steps of 1024
constexpr int kMaxTopkLarge = 8192;
constexpr int kTileKeys = 64;           // decode: minimum keys per segment
constexpr int kPipeKeys = 32;           // keys per K tile of the score pipelines (one MFMA column block)
constexpr int kDenseWaves = 4;          // dense prefill: 4 query rows per workgroup, 2 workgroups / CU
constexpr int kDecodeMaxRows = 4;       // decode mode: at most this many query rows per batch
constexpr int kDecodeWaves = 4;         // decode split kernel: waves per workgroup
constexpr int kDecodeSegments = 1024;   // decode: key segments per pass (256 CUs x 4 waves)
constexpr int kSelectThreads = 1024;    // decode-mode select kernel
constexpr int kSelectBuckets = 2048;    // decode-mode select: histogram buckets
constexpr size_t kLdsBudget = 160 * 1024;
constexpr int kDenseScratch = 512 * 4 + 4 * 64 * 4;  // dense kernel, rows in LDS: 512-bucket histogram + gather
constexpr int kListScratch = 320 * 4 + 4 * 64 * 4;   // dense kernel, candidate lists: merge-select scratch
// dense kernel, rows in global memory: 2048-bucket histogram, gather / rank scratch, select histogram
constexpr int kWideScratch = 2048 * 4 + 4 * 64 * 4 + 320 * 4;
constexpr int kListRoom = 6 * kPipeKeys;  // candidate lists: free slots at the start of a pipeline run
// Rows of up to this many keys keep their scores in a workspace row; longer
// rows stream through candidate lists (the list's merges are wave-serial
// selects over about k + cap entries, which pay off only for rows many times
// longer than k; measured: 16K-key rows run 1.4x faster with workspace rows,
// 128K-key rows 1.05x slower).
constexpr int kGlobalRowKeys = 32768;
constexpr int kDenseSlots = 512;         // resident dense workgroups: 2 per CU on 256 CUs
constexpr int kMetaMagic = 0x4C494D44;  // "LIMD"
// The workspace starts with a status block: int32 word 0 receives the call's
// status (0, or kStatusMetaMismatch when the metadata was built for another
// problem); the kernels' scratch follows it.
constexpr size_t kStatusBytes = 256;
constexpr int32_t kStatusMetaMismatch = 5;   // = LI_ERR_METADATA_MISMATCH

// kModeDense: rows of at most `dcap` keys, every score kept in LDS;
// kModeDenseGlobal: rows of up to kGlobalRowKeys keys, every score in a
// workspace row; kModeDenseList: longer rows, a running top-k in the output
// slots and an LDS candidate list per row; kModeDecode: a few query rows per
// batch, split keys.
enum Mode : int32_t { kModeDense = 0, kModeDenseGlobal = 1, kModeDecode = 2, kModeDenseList = 3 };
// Row modes of the dense kernel (where a row's scores go), one per prefill mode.
enum RowMode : int { kRowsLds = 0, kRowsGlobal = 1, kRowsList = 2 };

// Metadata buffer layout (all int32 / int4 records, offsets in bytes):
//   [0, 256)        header, see MetaHeader
//   batch table     B x int4 {q_tok_off, s1_b, k_tok_off, s2_b}
//   counts          B x int32  (items per batch)
//   starts          B x int32  (exclusive prefix of counts)
//   items           max_items x int4
//     prefill item: {b, q0, nrows, 0}
//     decode item : {b, i, k0, k1}
struct MetaHeader {
  int32_t n_items;
  int32_t mode;
  int32_t chunk;
  int32_t magic;
  int32_t batch;
  int32_t max_items;
  uint32_t fingerprint;   // of the li_problem the metadata was built for
  // the persistent prefill kernels' dynamic walk of the items: the next item to
  // take and the workgroups done; li_metadata zeroes both, and every such
  // kernel leaves them at zero when its last workgroup ends
  int32_t work_next;
  int32_t work_done;
  int32_t pad[55];
};
static_assert(sizeof(MetaHeader) == 256, "metadata header is 256 bytes");

struct Plan {
  int32_t mode;
  int32_t max_items;
  int32_t rows_per_item;  // prefill: query rows per work item
  int32_t chunk;          // decode: minimum keys per segment
  int32_t cap;            // candidate-list prefill: LDS list entries per row
  int32_t dcap;           // dense prefill: score slots per row
  int32_t mblocks;        // 1 (N1 <= 32) or 2 (N1 <= 64)
  size_t lds_prefill;     // dynamic LDS of the prefill kernel
  size_t lds_select;      // dynamic LDS of the decode-mode select kernel
  size_t meta_bytes;
  size_t off_batch, off_counts, off_starts, off_items;
  size_t ws_bytes;
  int64_t ws_row_stride;  // decode: fp32 slots per (batch, row) score row
  int32_t seg_mm_stride;  // decode: segment (min, max) pairs per row
  int32_t grid;           // candidate-list prefill: resident workgroups
};

// Kernel argument block (passed by value).
struct KArgs {
  const void* q;
  const void* k;
  const void* w;
  const float* q_descale;
  const float* k_descale;
  const int32_t* block_table;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* seqused_k;
  const int32_t* cmp_res;   // compressed keys under mask 3: residual original keys per batch
  const int32_t* idx_off;   // NULL or an index offset per batch
  unsigned char* meta;      // metadata base
  float* ws;                // decode: dense score rows; candidate lists: top-k values
                            // (when sparse_values is NULL), topk per resident wave
  float* seg_mm;            // decode: (min, max) score of each segment, seg_mm_stride pairs per row
  int32_t* out_idx;
  float* out_val;
  int32_t* status;          // workspace status word, or NULL (li_gather)
  int64_t k_block_stride_bytes;   // bytes between paged blocks
  int64_t ws_row_stride;
  int32_t seg_mm_stride;
  int32_t batch, s1max, s2max;
  int32_t n1, topk, cmp_ratio;
  int32_t layout_q, layout_k, mask_mode;
  int32_t block_size, block_shift, max_blocks_per_seq;
  int32_t cap, dcap, chunk, max_items, rows_per_item;
  int32_t off_batch, off_counts, off_starts, off_items;
  uint32_t fingerprint;     // of the problem of this call
  int32_t rows;             // query rows (B * S1, or T1)
};

// Layout / dtype codes as in li.h.
enum { L_BSND = 0, L_TND = 1, L_PA = 2 };
// How a kernel addresses K: contiguous tokens, a paged pool, or a paged pool
// whose block size is a multiple of 32 keys (a 32-key tile never spans blocks).
enum { KL_CONTIG = 0, KL_PAGED = 1, KL_PAGED_TILE = 2 };
enum { DT_BF16 = 0, DT_FP8 = 1, DT_FP32 = 2, DT_FP16 = 3 };

// li_gather: the selected rows' source and destination.
struct GatherArgs {
  const int32_t* idx;       // sparse_indices [rows, topk]
  unsigned char* out;       // [rows, topk * sel, row_bytes]
  int32_t row_bytes;        // bytes per token row, a multiple of 16
  int32_t sel;              // tokens per selected index
};
constexpr int kGatherRows = 64;          // selected rows per gather workgroup

// li_grad_kl: the backward of the indexer fused with its KL loss.
struct GradArgs {
  const void* q;            // main attention: [rows, G, 128]
  const void* k;            // [keys, 128]
  const void* q_rope;       // [rows, G, 64] or NULL
  const void* k_rope;       // [keys, 64] or NULL
  const void* qi;           // indexer: [rows, Ni, 128]
  const void* ki;           // [keys, 128]
  const void* w;            // [rows, Ni]
  const int32_t* sel;       // sparse_indices [rows, topk]
  const float* smax;        // softmax_max [rows, G]
  const float* ssum;        // softmax_sum [rows, G]
  const int32_t* cu_q;      // TND: inclusive prefix sums, else NULL
  const int32_t* cu_k;
  float* d_qi;              // [rows, Ni, 128]
  float* d_ki;              // [keys, 128]
  float* d_w;               // [rows, Ni]
  float* loss;              // [1]
  float* loss_rows;         // workspace: [rows]
  int64_t keys;
  int32_t rows, batch, s1, s2, layout;
  int32_t G, Ni, topk, topk_pad;
  float scale;
};
constexpr int kGradWaves = 4;            // rows per workgroup of the backward row kernel
constexpr int kGradTileBytes = 20480;    // per wave: index, main and rope key tiles

// Launchers (defined in the .hip files); return the hipGetLastError() of the launch.
hipError_t launch_metadata(const KArgs& a, int mode, hipStream_t s);
hipError_t launch_gather(const KArgs& a, const GatherArgs& g, int64_t rows, hipStream_t s);
hipError_t launch_prefill(const KArgs& a, int mode, int qk_dtype, int w_dtype, int mblocks,
                          int kl, int grid, size_t lds, hipStream_t s);
hipError_t launch_decode(const KArgs& a, int qk_dtype, int w_dtype, int mblocks, int kl,
                         int grid, hipStream_t s);
hipError_t launch_select(const KArgs& a, int grid, size_t lds, hipStream_t s);
size_t select_shared_bytes();   // LDS of the select kernel
hipError_t launch_grad(const GradArgs& g, int qk_dtype, int w_dtype, bool rope, hipStream_t s);

}  // namespace li
