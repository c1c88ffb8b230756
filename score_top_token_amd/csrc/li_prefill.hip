// Prefill launch: dispatch on the key dtype to its translation unit.
#include "li_internal.h"

namespace li {

hipError_t launch_prefill_bf16(const KArgs& a, int mode, int w_dtype, int mblocks, int kl, int grid,
                               size_t lds, hipStream_t s);
hipError_t launch_prefill_fp16(const KArgs& a, int mode, int w_dtype, int mblocks, int kl, int grid,
                               size_t lds, hipStream_t s);
hipError_t launch_prefill_fp8(const KArgs& a, int mode, int w_dtype, int mblocks, int kl, int grid,
                              size_t lds, hipStream_t s);

hipError_t launch_prefill(const KArgs& a, int mode, int qk_dtype, int w_dtype, int mblocks,
                          int kl, int grid, size_t lds, hipStream_t s) {
  switch (qk_dtype) {
    case DT_BF16: return launch_prefill_bf16(a, mode, w_dtype, mblocks, kl, grid, lds, s);
    case DT_FP16: return launch_prefill_fp16(a, mode, w_dtype, mblocks, kl, grid, lds, s);
    case DT_FP8: return launch_prefill_fp8(a, mode, w_dtype, mblocks, kl, grid, lds, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace li
