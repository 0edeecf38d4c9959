// Row-kernel instance: 32 elements per lane, 2-4 waves per row (2049-8192 columns).
// Its element passes take their elements in chunks of 16 (table reads in flight
// together): with the fixed-point bins this instance then spills nothing in the default
// path, against 16 bytes per lane with chunks of 8, and the rounds run ~2% faster.
#define ANY4_CHUNK 16
#include "any4_rows.h"

namespace any4 {
hipError_t launch_rows_e32_w8(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  return launch_mode<32, 8>(args, mode, n_blocks, stream);
}

}  // namespace any4
