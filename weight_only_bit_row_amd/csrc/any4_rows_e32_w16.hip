// Row-kernel instance: 32 elements per lane, up to 16 waves per row at up to 128 VGPRs (the
// 1024-lane instance): rows of 5-16 waves (8193-32768 columns), and on the default path
// also rows of 2-4 waves (2049-8192 columns), eight 2-wave rows per CU.
#include "any4_rows.h"

namespace any4 {
hipError_t launch_rows_e32_w16(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  return launch_mode<32, 16>(args, mode, n_blocks, stream);
}

}  // namespace any4
