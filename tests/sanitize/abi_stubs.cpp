// Host-only stand-ins for the kernel launchers and the two HIP runtime calls of the ABI
// layer, so that any4_api.cpp builds with g++ under AddressSanitizer and
// UndefinedBehaviorSanitizer and its validation, batching and workspace carving run on a
// machine without a GPU.  No stand-in dereferences a device pointer; the row-kernel
// launcher checks the batch layout that the kernel relies on and counts launches.
#include <hip/hip_runtime_api.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "any4_launch.h"

int g_row_launches = 0;
int64_t g_rows_launched = 0;

static void fail(const char* what) {
  std::fprintf(stderr, "stub check failed: %s\n", what);
  std::abort();
}

namespace any4 {

hipError_t launch_rows(const LaunchArgs& a, RowConfig cfg, int mode, int64_t n_blocks, hipStream_t) {
  if (n_blocks <= 0) return hipSuccess;
  if (a.n_mats < 1 || a.n_mats > kMaxMats) fail("n_mats");
  if (a.nw != cfg.nw || cfg.nw < 1 || cfg.nw > 16) fail("waves per row");
  if (mode < MODE_FULL || mode > MODE_STEP) fail("mode");
  if (a.row_start[0] != 0) fail("row_start[0]");
  for (int i = 0; i < a.n_mats; ++i) {
    if (a.row_start[i + 1] - a.row_start[i] != a.m[i].n_rows) fail("row_start spacing");
    if (choose_config(a.m[i].n_cols).nw != cfg.nw || choose_config(a.m[i].n_cols).e != cfg.e)
      fail("mixed geometry in one launch");
    if (mode == MODE_FULL && (!a.m[i].codes || !a.m[i].lut || !a.m[i].scale || !a.m[i].offset))
      fail("missing output");
  }
  for (int i = a.n_mats; i <= kMaxMats; ++i)
    if (a.row_start[i] != n_blocks) fail("row_start tail");
  if (n_blocks > INT32_MAX) fail("grid");
  ++g_row_launches;
  g_rows_launched += n_blocks;
  return hipSuccess;
}

hipError_t launch_clear_status(uint32_t* status, hipStream_t) { return status ? hipSuccess : hipErrorInvalidValue; }
hipError_t launch_copy_status(const uint32_t* src, uint32_t* dst, hipStream_t) {
  return (src && dst) ? hipSuccess : hipErrorInvalidValue;
}
hipError_t launch_pack(const MatDesc&, int, int, const uint8_t*, const float*, const float*, const float*,
                       hipStream_t) {
  return hipSuccess;
}
hipError_t launch_sorted_lloyd(SortedDesc d, hipStream_t) {
  if (d.n_cols < 2 || d.n_cols > 2 * kSortedMaxCols) return hipErrorInvalidValue;
  return (d.n_cols <= kSortedMaxCols || d.work) ? hipSuccess : hipErrorInvalidValue;
}
size_t sorted_lloyd_work_bytes(int64_t n_rows, int64_t n_cols) {
  return n_cols > kSortedMaxCols ? static_cast<size_t>(n_rows) * 3 * sizeof(float) * kSortedMaxCols : 0;
}
hipError_t launch_restart_merge(const MergeDesc& d, hipStream_t) {
  return (d.cand_codes && d.codes && d.best_obj) ? hipSuccess : hipErrorInvalidValue;
}
AbsmeanPlan plan_absmean(int64_t n_tokens, int64_t n_cols) {
  AbsmeanPlan p;
  p.n_splits = n_tokens > 256 ? 2 : 1;
  p.tokens_per_split = (n_tokens + p.n_splits - 1) / p.n_splits;
  p.partial_bytes = size_t(p.n_splits) * size_t(n_cols) * sizeof(double);
  return p;
}
hipError_t launch_absmean(const void*, int, int64_t, int64_t, float*, double*, const AbsmeanPlan&, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_dequant(const DequantDesc&, hipStream_t) { return hipSuccess; }
hipError_t launch_gemv(const GemvDesc&, hipStream_t) { return hipSuccess; }

// the scratch of the entry point that allocates nothing: an address the stand-ins never
// dereference
hipError_t noalloc_scratch(unsigned char** out) {
  static unsigned char host_stand_in[256];
  *out = host_stand_in;
  return hipSuccess;
}

}  // namespace any4

hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipMemcpy(void* dst, const void*, size_t n, hipMemcpyKind) {
  std::memset(dst, 0, n);
  return hipSuccess;
}
