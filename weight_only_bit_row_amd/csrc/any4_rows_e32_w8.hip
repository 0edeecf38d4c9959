// Row-kernel instance: 32 elements per lane, 2-4 waves per row (2049-8192 columns).
#include "any4_rows.h"

namespace any4 {
hipError_t launch_rows_e32_w8(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  return launch_mode<32, 8>(args, mode, n_blocks, stream);
}

}  // namespace any4
