// Row-kernel instance: 8 elements per lane, one wave per row (rows of at most 512 columns).
#include "any4_rows.h"

namespace any4 {
hipError_t launch_rows_e8(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  return launch_mode<8, 1>(args, mode, n_blocks, stream);
}

}  // namespace any4
