// Row-kernel instance: 32 elements per lane, 5-16 waves per row (8193-32768 columns).
#include "any4_rows.h"

namespace any4 {
hipError_t launch_rows_e32_w16(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  return launch_mode<32, 16>(args, mode, n_blocks, stream);
}

}  // namespace any4
