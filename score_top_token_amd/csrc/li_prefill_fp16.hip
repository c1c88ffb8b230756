// Prefill kernels for fp16 keys: the instances of the templates in
// li_prefill_kernels.h for one key dtype (the dtypes compile side by side).
#include "li_prefill_kernels.h"

namespace li {

hipError_t launch_prefill_fp16(const KArgs& a, int mode, int w_dtype, int mblocks, int kl, int grid,
                             size_t lds, hipStream_t s) {
  return launch_mb<DT_FP16>(a, mode, w_dtype, mblocks, kl, grid, lds, s);
}

}  // namespace li
