// Row-kernel instance: 32 elements per lane, one wave per row (1025-2048 columns).
#include "any4_rows.h"

namespace any4 {
hipError_t launch_rows_e32_w1(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  return launch_mode<32, 1>(args, mode, n_blocks, stream);
}

}  // namespace any4
