// Row-kernel instance: 16 elements per lane, one wave per row (513-1024 columns).
#include "any4_rows.h"

namespace any4 {
hipError_t launch_rows_e16(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  return launch_mode<16, 1>(args, mode, n_blocks, stream);
}

}  // namespace any4
