// Internal interface between the C-ABI layer (any4_api.cpp) and the gfx950 kernels
// (any4_kernels.hip).  Not installed; the public interface is include/any4.h.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace any4 {

constexpr int kMaxMats = 8;       // matrices per launch (descriptors travel as kernel arguments)
constexpr int kMaxClusters = 16;
constexpr int kMaxCols = 32768;   // 16 waves x 64 lanes x 32 elements held in registers

enum Mode : int { MODE_FULL = 0, MODE_SCALE = 1, MODE_SEED = 2, MODE_STEP = 3 };

struct MatDesc {
  const void* w;
  const float* act;
  int64_t n_rows;
  int64_t n_cols;
  int64_t row_offset;
  int32_t dtype;
  int32_t matrix_index;
  // products
  uint8_t* codes;
  uint16_t* lut;
  uint16_t* scale;
  uint16_t* offset;
  double* objective;
  // stage inputs / outputs (NULL unless a stage entry point sets them)
  float* ws_out;
  float* alpha_out;
  float* beta_out;
  float* a_out;
  const float* c_in;
  float* c_out;
  uint8_t* assign_out;
  int32_t* picks_out;
};

// Method variant word (any4_params.variant; 0 = the paper's defaults).
constexpr int32_t kVarWeightMask = 0x3;       // sample weights: 0 alpha*E|x|, 1 E|x|, 2 none
constexpr int32_t kVarInitShift = 2;          // init: 0 k-means++, 1 random, 2 uniform levels
constexpr int32_t kVarSymmetric = 1 << 4;     // Eq. 3 scaling
constexpr int32_t kVarAllRounds = 1 << 5;     // no stop at a fixed point (not a method variant)
constexpr int32_t kVarRestartShift = 8;       // bits 8-15: restarts - 1
constexpr int32_t kVarKnownBits = 0xFF3F;
enum : int32_t { INIT_KMEANSPP = 0, INIT_RANDOM = 1, INIT_UNIFORM = 2, INIT_GREEDY = 3 };

struct LaunchArgs {
  MatDesc m[kMaxMats];
  int64_t row_start[kMaxMats + 1];  // block b belongs to matrix i when row_start[i] <= b < row_start[i+1]
  int32_t n_mats;
  int32_t group;
  int32_t n_clusters;
  int32_t iters;
  int32_t nw;                       // waves per row (one workgroup per row)
  int32_t variant;                  // method variant word (restart bits are handled by the host)
  uint64_t seed;
  uint32_t* status;                 // device status word or NULL
  int32_t restart;                  // the Philox counter's second word is t + 16 * restart
  int32_t all_rounds;               // run every round, no stop at an exact fixed point
};

// Row-kernel launch geometry for a row length: elements per lane E and waves per row.
struct RowConfig {
  int e;
  int nw;
};
RowConfig choose_config(int64_t n_cols);  // any4_api.cpp

// Row-kernel instances, one translation unit each (any4_rows_e*.hip): 8 or 16
// elements per lane on one wave, 32 on one wave, 2-4 waves, and 5-16 waves.
hipError_t launch_rows_e8(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream);
hipError_t launch_rows_e16(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream);
hipError_t launch_rows_e32_w1(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream);
hipError_t launch_rows_e32_w8(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream);
hipError_t launch_rows_e32_w16(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream);
// Launch one row kernel over all rows of args (args.nw must match cfg.nw).
hipError_t launch_rows(const LaunchArgs& args, RowConfig cfg, int mode, int64_t n_blocks,
                       hipStream_t stream);
// Clear the status word (a one-thread kernel: no memset node is recorded).
hipError_t launch_clear_status(uint32_t* status, hipStream_t stream);
// Copy the status word to a caller's buffer (a one-thread kernel).
hipError_t launch_copy_status(const uint32_t* src, uint32_t* dst, hipStream_t stream);

// Library-owned scratch of any4_quantize_noalloc: kNoallocScratchBytes of device memory per
// device (a static device array), its address on the current device looked up on first use.
constexpr size_t kNoallocScratchBytes = size_t(32) << 20;
hipError_t noalloc_scratch(unsigned char** out);
// Emission-only kernel behind any4_stage_pack.
hipError_t launch_pack(const MatDesc& m, int group, int n_clusters, const uint8_t* assign,
                       const float* c, const float* alpha, const float* beta, hipStream_t stream);

// Sorted-row Lloyd rounds behind any4_stage_lloyd_sorted: from the scaled rows w_s and
// sample weights a ([n_rows, n_cols] fp32 each) and the centroids c_in [n_rows, k], run
// `iters` rounds and write c_out [n_rows, k].  One 256-lane workgroup per row, the row
// sorted in LDS (8 bytes per padded column: 128 KB at 16384) for rows of at most
// kSortedMaxCols columns; longer rows, up to twice that, are sorted as two halves in turn
// and keep their sorted sample weights in `work` (sorted_lloyd_work_bytes).
constexpr int kSortedMaxCols = 16384;
struct SortedDesc {
  const float* w_s;
  const float* a;
  const float* c_in;
  float* c_out;
  float* work;         // rows past kSortedMaxCols: 3 x kSortedMaxCols floats per row
  int64_t n_rows;
  int32_t n_cols;
  int32_t kp;          // n_cols rounded up to a power of two (set by the launcher)
  int32_t n_clusters;
  int32_t iters;
  int32_t symmetric;   // symmetric scaling: w_S in [-k/2, k/2]
  int32_t pad_;
};
size_t sorted_lloyd_lds_bytes(int64_t n_cols);
size_t sorted_lloyd_work_bytes(int64_t n_rows, int64_t n_cols);
hipError_t launch_sorted_lloyd(SortedDesc d, hipStream_t stream);

// Restarts: after restart r has written its outputs to the `cand_*` buffers, keep them
// for every row whose objective is below the best so far (the earlier restart wins ties).
struct MergeDesc {
  int64_t n_rows;
  int64_t n_cols;
  int32_t n_clusters;
  int32_t pad_;
  const uint8_t* cand_codes;
  const uint16_t* cand_lut;
  const double* cand_obj;
  const float* cand_c;        // or NULL
  const int32_t* cand_picks;  // or NULL
  uint8_t* codes;
  uint16_t* lut;
  double* best_obj;
  float* c;                   // or NULL
  int32_t* picks;             // or NULL
};
hipError_t launch_restart_merge(const MergeDesc& d, hipStream_t stream);

// ---- bookends (any4_bookends.hip)

// E|x_j| reduction: token slices of the [T, K] batch and the fp64 partial sums they need.
struct AbsmeanPlan {
  int64_t n_splits;          // token slices, each summed on its own
  int64_t tokens_per_split;
  size_t partial_bytes;      // n_splits * K fp64 partial sums
};
AbsmeanPlan plan_absmean(int64_t n_tokens, int64_t n_cols);
hipError_t launch_absmean(const void* x, int dtype, int64_t n_tokens, int64_t n_cols, float* out,
                          double* partial, const AbsmeanPlan& plan, hipStream_t stream);

// Eq. 4 dequantization of one matrix's emitted codes/LUT/scale/offset.
struct DequantDesc {
  const uint8_t* codes;
  const uint16_t* lut;
  const uint16_t* scale;
  const uint16_t* offset;
  void* out;
  int64_t n_rows;
  int64_t n_cols;
  int32_t group;
  int32_t n_clusters;
  int32_t out_bf16;          // 0: fp32 output, 1: bf16 (round to nearest even)
  int32_t pad_;
};
hipError_t launch_dequant(const DequantDesc& d, hipStream_t stream);

// y [M, N] fp32 = x [M, K] times the Eq. 4 dequantized weight, transposed (M <= 8).
struct GemvDesc {
  const uint8_t* codes;
  const uint16_t* lut;
  const uint16_t* scale;
  const uint16_t* offset;
  const void* x;
  float* y;
  int64_t n_tokens;          // M
  int64_t n_rows;            // N
  int64_t n_cols;            // K
  int32_t group;
  int32_t n_clusters;
  int32_t x_bf16;            // 0: fp32 x, 1: bf16 bits
  int32_t pad_;
};
constexpr int kGemvMaxTokens = 8;
// token counts from which bf16 activations use the matrix-core kernel (measured)
constexpr int kGemvMfmaMinTokens = 3;
hipError_t launch_gemv(const GemvDesc& d, hipStream_t stream);

}  // namespace any4
