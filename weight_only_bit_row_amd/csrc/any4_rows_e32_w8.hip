// Row-kernel instance: 32 elements per lane, 2-4 waves per row (2049-8192 columns), at
// up to 168 VGPRs; rows with a method variant run here (the default path's rows of 2-4
// waves run on the 1024-lane instance).  Its element passes take their elements in
// chunks of 16 (table reads in flight together): with the fixed-point bins the default
// instance then spills nothing, against 16 bytes per lane with chunks of 8.
#define ANY4_CHUNK 16
#include "any4_rows.h"

namespace any4 {
hipError_t launch_rows_e32_w8(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  return launch_mode<32, 8>(args, mode, n_blocks, stream);
}

}  // namespace any4
