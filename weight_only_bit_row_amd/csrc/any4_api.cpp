// C ABI of the any4 quantizer (declared in include/any4.h): argument validation,
// batching of matrices into row-kernel launches, and the stage entry points.
// Everything here runs on the host and only enqueues work on the caller's stream.
#include "any4.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "any4_launch.h"

namespace any4 {

// Launch geometry for a row length, from measurements: 32 elements per lane (several
// waves per row) beat one 64-element wave per row on 14336 x 4096, whose register file
// allows only one wave per SIMD.  Rows longer than 16384 keep 32 elements per lane on up
// to 16 waves: against 64 elements on up to 8 waves (256 VGPRs, more spilled) they took
// 7.7 ms instead of 8.3 on 8192 x 28672 and 3.0 instead of 3.9 on 4096 x 20480, with the
// same output bits.
RowConfig choose_config(int64_t K) {
  if (K <= 512) return {8, 1};
  if (K <= 1024) return {16, 1};
  return {32, static_cast<int>((K + 2047) / 2048)};
}

}  // namespace any4

namespace {

using any4::LaunchArgs;
using any4::MatDesc;
using any4::RowConfig;

constexpr size_t kWorkspaceBytes = 256;

bool is_pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

int check_params(const any4_params* p) {
  if (!p) return ANY4_ERR_INVALID_ARG;
  if (p->group < 2 || !is_pow2(p->group)) return ANY4_ERR_INVALID_ARG;
  if (!(p->n_clusters == 2 || p->n_clusters == 4 || p->n_clusters == 8 || p->n_clusters == 16))
    return ANY4_ERR_INVALID_ARG;
  if (p->iters < 0) return ANY4_ERR_INVALID_ARG;
  if ((p->variant & ~any4::kVarKnownBits) != 0) return ANY4_ERR_INVALID_ARG;
  if ((p->variant & any4::kVarWeightMask) == 3) return ANY4_ERR_INVALID_ARG;
  return ANY4_OK;
}

int restarts_of(const any4_params* p) { return ((p->variant >> any4::kVarRestartShift) & 0xFF) + 1; }

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

// Workspace carved per matrix for restarts > 1: a candidate restart's codes, LUT,
// objective, fp32 centroids and picks, and the best objective so far.
struct RestartBufs {
  uint8_t* codes;
  uint16_t* lut;
  double* obj;
  float* c;
  int32_t* picks;
  double* best_obj;
};

size_t restart_bytes(const any4_matrix* m, int k) {
  const size_t n = static_cast<size_t>(m->n_rows);
  return align256(n * static_cast<size_t>(m->n_cols / 2)) + align256(n * k * 2) +
         2 * align256(n * 8) + 2 * align256(n * k * 4);
}

RestartBufs carve_restart(unsigned char*& base, const any4_matrix* m, int k) {
  const size_t n = static_cast<size_t>(m->n_rows);
  RestartBufs b;
  b.codes = base;
  base += align256(n * static_cast<size_t>(m->n_cols / 2));
  b.lut = reinterpret_cast<uint16_t*>(base);
  base += align256(n * k * 2);
  b.obj = reinterpret_cast<double*>(base);
  base += align256(n * 8);
  b.c = reinterpret_cast<float*>(base);
  base += align256(n * k * 4);
  b.picks = reinterpret_cast<int32_t*>(base);
  base += align256(n * k * 4);
  b.best_obj = reinterpret_cast<double*>(base);
  base += align256(n * 8);
  return b;
}

int check_matrix(const any4_matrix* m, const any4_params* p, bool need_products) {
  if (!m) return ANY4_ERR_INVALID_ARG;
  if (m->n_rows < 0 || m->n_cols < 2 || (m->n_cols & 1)) return ANY4_ERR_INVALID_ARG;
  if (m->n_cols % p->group != 0) return ANY4_ERR_INVALID_ARG;
  if (m->w_dtype != ANY4_F32 && m->w_dtype != ANY4_BF16) return ANY4_ERR_INVALID_ARG;
  if (m->row_offset < 0 || m->row_offset > INT64_MAX - m->n_rows) return ANY4_ERR_INVALID_ARG;
  if (m->n_cols > any4::kMaxCols) return ANY4_ERR_UNSUPPORTED;
  if (m->n_rows > INT32_MAX) return ANY4_ERR_UNSUPPORTED;
  if (m->n_rows == 0) return ANY4_OK;
  if (!m->w || !m->act_absmean) return ANY4_ERR_INVALID_ARG;
  if (need_products && (!m->codes || !m->lut || !m->scale || !m->offset))
    return ANY4_ERR_INVALID_ARG;
  return ANY4_OK;
}

MatDesc make_desc(const any4_matrix* m) {
  MatDesc d;
  std::memset(&d, 0, sizeof(d));
  d.w = m->w;
  d.act = m->act_absmean;
  d.n_rows = m->n_rows;
  d.n_cols = m->n_cols;
  d.row_offset = m->row_offset;
  d.dtype = m->w_dtype;
  d.matrix_index = m->matrix_index;
  d.codes = m->codes;
  d.lut = m->lut;
  d.scale = m->scale;
  d.offset = m->offset;
  d.objective = m->objective;
  return d;
}

LaunchArgs make_args(const any4_params* p, int nw, uint32_t* status) {
  LaunchArgs a;
  std::memset(&a, 0, sizeof(a));
  a.group = p->group;
  a.n_clusters = p->n_clusters;
  a.iters = p->iters;
  a.nw = nw;
  a.variant = p->variant & ((1 << any4::kVarRestartShift) - 1) & ~any4::kVarAllRounds;
  a.all_rounds = (p->variant & any4::kVarAllRounds) ? 1 : 0;
  a.restart = 0;
  a.seed = p->seed;
  a.status = status;
  return a;
}

int launch_one(const LaunchArgs& base, const MatDesc& d, int mode, hipStream_t stream) {
  if (d.n_rows == 0) return ANY4_OK;
  const RowConfig cfg = any4::choose_config(d.n_cols);
  LaunchArgs a = base;
  a.nw = cfg.nw;
  a.m[0] = d;
  a.n_mats = 1;
  a.row_start[0] = 0;
  for (int i = 1; i <= any4::kMaxMats; ++i) a.row_start[i] = d.n_rows;
  const hipError_t e = any4::launch_rows(a, cfg, mode, d.n_rows, stream);
  return e == hipSuccess ? ANY4_OK : ANY4_ERR_HIP;
}

int validate_batch(const any4_matrix* mats, int32_t count, const any4_params* p) {
  int st = check_params(p);
  if (st != ANY4_OK) return st;
  if (count < 0 || (count > 0 && !mats)) return ANY4_ERR_INVALID_ARG;
  for (int32_t i = 0; i < count; ++i) {
    st = check_matrix(&mats[i], p, true);
    if (st != ANY4_OK) return st;
  }
  return ANY4_OK;
}


// The batched path: every matrix of the batch through the row kernel, matrices of one
// row geometry in one launch (up to kMaxMats each), longer rows first so that the
// longest blocks start earliest.  Restart r (Philox counters t + 16 r): the first writes
// the outputs, each later one writes candidates into the workspace that replace a row's
// outputs where its objective is lower.  c_final / picks: optional per-matrix device
// arrays (or NULL) for the fp32 centroids and the k-means++ picks of the kept run.
// `order` and `rb` are caller storage for `count` entries; arguments are validated and
// the workspace is at least workspace_bytes_for() large.  in_place_sort orders the
// matrices without heap memory (for the entry point that allocates nothing).
int quantize_core(const any4_matrix* mats, int32_t count, const any4_params* params,
                  float* const* c_final, int32_t* const* picks, unsigned char* workspace,
                  hipStream_t stream, int32_t* order, RestartBufs* rb, bool in_place_sort) {
  uint32_t* status = reinterpret_cast<uint32_t*>(workspace);
  if (any4::launch_clear_status(status, stream) != hipSuccess) return ANY4_ERR_HIP;
  const int R = restarts_of(params);
  const int k = params->n_clusters;
  if (R > 1) {
    unsigned char* base = workspace + kWorkspaceBytes;
    for (int32_t i = 0; i < count; ++i) rb[i] = carve_restart(base, &mats[i], k);
  }
  int32_t n_order = 0;
  for (int32_t i = 0; i < count; ++i)
    if (mats[i].n_rows > 0) order[n_order++] = i;
  if (!in_place_sort) {
    std::stable_sort(order, order + n_order, [&](int32_t x, int32_t y) {
      return mats[x].n_cols > mats[y].n_cols;
    });
  } else {
    // the same stable order by insertion, which takes no heap memory
    for (int32_t a = 1; a < n_order; ++a) {
      const int32_t v = order[a];
      int32_t b = a;
      for (; b > 0 && mats[order[b - 1]].n_cols < mats[v].n_cols; --b) order[b] = order[b - 1];
      order[b] = v;
    }
  }
  auto cf = [&](int32_t i) { return c_final ? c_final[i] : nullptr; };
  auto pk = [&](int32_t i) { return picks ? picks[i] : nullptr; };
  for (int r = 0; r < R; ++r) {
    int32_t i = 0;
    while (i < n_order) {
      const RowConfig cfg = any4::choose_config(mats[order[i]].n_cols);
      LaunchArgs a = make_args(params, cfg.nw, status);
      a.restart = r;
      int64_t rows = 0;
      a.n_mats = 0;
      while (i < n_order && a.n_mats < any4::kMaxMats) {
        const RowConfig c2 = any4::choose_config(mats[order[i]].n_cols);
        if (c2.e != cfg.e || c2.nw != cfg.nw) break;
        if (rows + mats[order[i]].n_rows > INT32_MAX) break;
        const int32_t mi = order[i];
        const any4_matrix* m = &mats[mi];
        MatDesc d = make_desc(m);
        d.c_out = cf(mi);
        d.picks_out = pk(mi);
        if (R > 1) {
          const RestartBufs& b = rb[mi];
          double* best = m->objective ? m->objective : b.best_obj;
          if (r == 0) {
            d.objective = best;
          } else {
            d.codes = b.codes;
            d.lut = b.lut;
            d.objective = b.obj;
            d.c_out = cf(mi) ? b.c : nullptr;
            d.picks_out = pk(mi) ? b.picks : nullptr;
          }
        }
        a.row_start[a.n_mats] = rows;
        a.m[a.n_mats] = d;
        rows += m->n_rows;
        ++a.n_mats;
        ++i;
      }
      for (int j = a.n_mats; j <= any4::kMaxMats; ++j) a.row_start[j] = rows;
      if (any4::launch_rows(a, cfg, any4::MODE_FULL, rows, stream) != hipSuccess)
        return ANY4_ERR_HIP;
    }
    if (r == 0) continue;
    for (int32_t oi = 0; oi < n_order; ++oi) {
      const int32_t mi = order[oi];
      const any4_matrix* m = &mats[mi];
      const RestartBufs& b = rb[mi];
      any4::MergeDesc md;
      std::memset(&md, 0, sizeof(md));
      md.n_rows = m->n_rows;
      md.n_cols = m->n_cols;
      md.n_clusters = k;
      md.cand_codes = b.codes;
      md.cand_lut = b.lut;
      md.cand_obj = b.obj;
      md.cand_c = cf(mi) ? b.c : nullptr;
      md.cand_picks = pk(mi) ? b.picks : nullptr;
      md.codes = m->codes;
      md.lut = m->lut;
      md.best_obj = m->objective ? m->objective : b.best_obj;
      md.c = cf(mi);
      md.picks = pk(mi);
      if (any4::launch_restart_merge(md, stream) != hipSuccess) return ANY4_ERR_HIP;
    }
  }
  return ANY4_OK;
}

size_t workspace_bytes_for(const any4_matrix* mats, int32_t count, const any4_params* params) {
  size_t bytes = kWorkspaceBytes;
  if (restarts_of(params) > 1)
    for (int32_t i = 0; i < count; ++i) bytes += restart_bytes(&mats[i], params->n_clusters);
  return bytes;
}

// Validation, workspace check and host storage for the batched path.
int quantize_checked(const any4_matrix* mats, int32_t count, const any4_params* params,
                     float* const* c_final, int32_t* const* picks, void* workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  const int st = validate_batch(mats, count, params);
  if (st != ANY4_OK) return st;
  if (!workspace || workspace_bytes < workspace_bytes_for(mats, count, params))
    return ANY4_ERR_WORKSPACE;
  std::vector<int32_t> order(static_cast<size_t>(count));
  std::vector<RestartBufs> rb(static_cast<size_t>(count));
  return quantize_core(mats, count, params, c_final, picks, static_cast<unsigned char*>(workspace),
                       stream, order.data(), rb.data(), false);
}

}  // namespace

extern "C" {

const char* any4_status_string(int status) {
  switch (status) {
    case ANY4_OK: return "ok";
    case ANY4_ERR_INVALID_ARG: return "invalid argument";
    case ANY4_ERR_UNSUPPORTED: return "unsupported shape or option";
    case ANY4_ERR_WORKSPACE: return "workspace missing or too small";
    case ANY4_ERR_HIP: return "HIP launch or runtime error";
    case ANY4_ERR_NONFINITE: return "a row held a non-finite or out-of-range value";
    default: return "unknown status";
  }
}

int any4_launch_geometry(int64_t n_cols, int32_t* elems_per_lane, int32_t* waves_per_row) {
  if (!elems_per_lane || !waves_per_row || n_cols < 2 || n_cols > any4::kMaxCols)
    return ANY4_ERR_INVALID_ARG;
  const RowConfig cfg = any4::choose_config(n_cols);
  *elems_per_lane = cfg.e;
  *waves_per_row = cfg.nw;
  return ANY4_OK;
}

int any4_workspace_bytes(const any4_matrix* mats, int32_t count, const any4_params* params,
                         size_t* bytes_out) {
  if (!bytes_out) return ANY4_ERR_INVALID_ARG;
  const int st = validate_batch(mats, count, params);
  if (st != ANY4_OK) return st;
  *bytes_out = workspace_bytes_for(mats, count, params);
  return ANY4_OK;
}

int any4_quantize(const any4_matrix* mats, int32_t count, const any4_params* params,
                  void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return quantize_checked(mats, count, params, nullptr, nullptr, workspace, workspace_bytes, stream);
}

int any4_stage_quantize_batch(const any4_matrix* mats, int32_t count, const any4_params* params,
                              float* const* c_final, int32_t* const* picks, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  return quantize_checked(mats, count, params, c_final, picks, workspace, workspace_bytes, stream);
}

int any4_quantize_noalloc(const any4_matrix* mats, int32_t count, const any4_params* params,
                          uint32_t* status_out, hipStream_t stream) {
  const int st = validate_batch(mats, count, params);
  if (st != ANY4_OK) return st;
  if (count > ANY4_NOALLOC_MAX_MATRICES) return ANY4_ERR_UNSUPPORTED;
  static_assert(ANY4_NOALLOC_SCRATCH_BYTES == any4::kNoallocScratchBytes, "scratch size");
  if (workspace_bytes_for(mats, count, params) > any4::kNoallocScratchBytes) return ANY4_ERR_WORKSPACE;
  unsigned char* scratch = nullptr;
  if (any4::noalloc_scratch(&scratch) != hipSuccess) return ANY4_ERR_HIP;
  int32_t order[ANY4_NOALLOC_MAX_MATRICES];
  RestartBufs rb[ANY4_NOALLOC_MAX_MATRICES];
  const int r = quantize_core(mats, count, params, nullptr, nullptr, scratch, stream, order, rb, true);
  if (r != ANY4_OK) return r;
  if (status_out &&
      any4::launch_copy_status(reinterpret_cast<const uint32_t*>(scratch), status_out, stream) != hipSuccess)
    return ANY4_ERR_HIP;
  return ANY4_OK;
}

int any4_read_device_status(const void* workspace, hipStream_t stream) {
  if (!workspace) return ANY4_ERR_WORKSPACE;
  if (hipStreamSynchronize(stream) != hipSuccess) return ANY4_ERR_HIP;
  uint32_t st = 0;
  if (hipMemcpy(&st, workspace, sizeof(st), hipMemcpyDeviceToHost) != hipSuccess)
    return ANY4_ERR_HIP;
  return st == 0 ? ANY4_OK : static_cast<int>(st);
}

int any4_stage_scale(const any4_matrix* m, const any4_params* params, float* w_s, float* alpha,
                     float* beta, float* a, hipStream_t stream) {
  int st = check_params(params);
  if (st == ANY4_OK) st = check_matrix(m, params, false);
  if (st != ANY4_OK) return st;
  if (m->n_rows > 0 && (!w_s || !alpha || !beta || !a)) return ANY4_ERR_INVALID_ARG;
  MatDesc d = make_desc(m);
  d.ws_out = w_s;
  d.alpha_out = alpha;
  d.beta_out = beta;
  d.a_out = a;
  return launch_one(make_args(params, 1, nullptr), d, any4::MODE_SCALE, stream);
}

int any4_stage_seed(const any4_matrix* m, const any4_params* params, float* c0, int32_t* picks,
                    hipStream_t stream) {
  int st = check_params(params);
  if (st == ANY4_OK) st = check_matrix(m, params, false);
  if (st != ANY4_OK) return st;
  if (m->n_rows > 0 && (!c0 || !picks)) return ANY4_ERR_INVALID_ARG;
  MatDesc d = make_desc(m);
  d.c_out = c0;
  d.picks_out = picks;
  return launch_one(make_args(params, 1, nullptr), d, any4::MODE_SEED, stream);
}

int any4_stage_lloyd_step(const any4_matrix* m, const any4_params* params, const float* c_in,
                          uint8_t* assign, float* c_out, double* objective, hipStream_t stream) {
  int st = check_params(params);
  if (st == ANY4_OK) st = check_matrix(m, params, false);
  if (st != ANY4_OK) return st;
  if (m->n_rows > 0 && (!c_in || !assign || !c_out)) return ANY4_ERR_INVALID_ARG;
  MatDesc d = make_desc(m);
  d.c_in = c_in;
  d.assign_out = assign;
  d.c_out = c_out;
  d.objective = objective;
  return launch_one(make_args(params, 1, nullptr), d, any4::MODE_STEP, stream);
}

int any4_stage_lloyd_sorted_workspace_bytes(int64_t n_rows, int64_t n_cols, size_t* bytes_out) {
  if (!bytes_out || n_rows < 0 || n_cols < 2 || (n_cols & 1)) return ANY4_ERR_INVALID_ARG;
  if (n_cols > 2 * static_cast<int64_t>(any4::kSortedMaxCols) || n_rows > INT32_MAX) return ANY4_ERR_UNSUPPORTED;
  *bytes_out = any4::sorted_lloyd_work_bytes(n_rows, n_cols);
  return ANY4_OK;
}

int any4_stage_lloyd_sorted(const any4_matrix* m, const any4_params* params, const float* w_s,
                            const float* a, const float* c_in, float* c_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  const int st = check_params(params);
  if (st != ANY4_OK) return st;
  if (!m || m->n_rows < 0 || m->n_cols < 2 || (m->n_cols & 1)) return ANY4_ERR_INVALID_ARG;
  if (m->n_cols > 2 * static_cast<int64_t>(any4::kSortedMaxCols) || m->n_rows > INT32_MAX)
    return ANY4_ERR_UNSUPPORTED;
  if (m->n_rows == 0) return ANY4_OK;
  if (!w_s || !a || !c_in || !c_out) return ANY4_ERR_INVALID_ARG;
  const size_t need = any4::sorted_lloyd_work_bytes(m->n_rows, m->n_cols);
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 15)))
    return ANY4_ERR_WORKSPACE;
  any4::SortedDesc d{};
  d.w_s = w_s;
  d.a = a;
  d.c_in = c_in;
  d.c_out = c_out;
  d.work = need > 0 ? static_cast<float*>(workspace) : nullptr;
  d.n_rows = m->n_rows;
  d.n_cols = static_cast<int32_t>(m->n_cols);
  d.n_clusters = params->n_clusters;
  d.iters = params->iters;
  d.symmetric = (params->variant & any4::kVarSymmetric) ? 1 : 0;
  return any4::launch_sorted_lloyd(d, stream) == hipSuccess ? ANY4_OK : ANY4_ERR_HIP;
}

int any4_stage_pack(const any4_matrix* m, const any4_params* params, const uint8_t* assign,
                    const float* c, const float* alpha, const float* beta, hipStream_t stream) {
  int st = check_params(params);
  if (st == ANY4_OK) st = check_matrix(m, params, false);
  if (st != ANY4_OK) return st;
  if (m->n_rows == 0) return ANY4_OK;
  if (!m->codes || !m->lut || !m->scale || !m->offset || !assign || !c || !alpha || !beta)
    return ANY4_ERR_INVALID_ARG;
  const MatDesc d = make_desc(m);
  return any4::launch_pack(d, params->group, params->n_clusters, assign, c, alpha, beta,
                           stream) == hipSuccess
             ? ANY4_OK
             : ANY4_ERR_HIP;
}

int any4_stage_full(const any4_matrix* m, const any4_params* params, float* c_final,
                    int32_t* picks, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return quantize_checked(m, 1, params, &c_final, &picks, workspace, workspace_bytes, stream);
}

int any4_act_absmean_workspace_bytes(int64_t n_tokens, int64_t n_cols, size_t* bytes_out) {
  if (!bytes_out || n_tokens < 1 || n_cols < 1) return ANY4_ERR_INVALID_ARG;
  *bytes_out = any4::plan_absmean(n_tokens, n_cols).partial_bytes;
  return ANY4_OK;
}

int any4_act_absmean(const void* x, int32_t x_dtype, int64_t n_tokens, int64_t n_cols,
                     float* act_absmean, void* workspace, size_t workspace_bytes,
                     hipStream_t stream) {
  if (!x || !act_absmean || n_tokens < 1 || n_cols < 1) return ANY4_ERR_INVALID_ARG;
  if (x_dtype != ANY4_F32 && x_dtype != ANY4_BF16) return ANY4_ERR_INVALID_ARG;
  const any4::AbsmeanPlan plan = any4::plan_absmean(n_tokens, n_cols);
  if (!workspace || workspace_bytes < plan.partial_bytes) return ANY4_ERR_WORKSPACE;
  return any4::launch_absmean(x, x_dtype, n_tokens, n_cols, act_absmean,
                              static_cast<double*>(workspace), plan, stream) == hipSuccess
             ? ANY4_OK
             : ANY4_ERR_HIP;
}

int any4_dequantize(const any4_matrix* m, const any4_params* params, void* w_out,
                    int32_t out_dtype, hipStream_t stream) {
  if (!m || !params) return ANY4_ERR_INVALID_ARG;
  if (params->group < 2 || !is_pow2(params->group)) return ANY4_ERR_INVALID_ARG;
  if (!(params->n_clusters == 2 || params->n_clusters == 4 || params->n_clusters == 8 ||
        params->n_clusters == 16))
    return ANY4_ERR_INVALID_ARG;
  if (m->n_rows < 0 || m->n_cols < 2 || (m->n_cols & 1) || m->n_cols % params->group != 0)
    return ANY4_ERR_INVALID_ARG;
  if (out_dtype != ANY4_F32 && out_dtype != ANY4_BF16) return ANY4_ERR_INVALID_ARG;
  if (m->n_rows > INT32_MAX) return ANY4_ERR_UNSUPPORTED;
  if (m->n_rows == 0) return ANY4_OK;
  if (!m->codes || !m->lut || !m->scale || !m->offset || !w_out) return ANY4_ERR_INVALID_ARG;
  any4::DequantDesc d;
  std::memset(&d, 0, sizeof(d));
  d.codes = m->codes;
  d.lut = m->lut;
  d.scale = m->scale;
  d.offset = m->offset;
  d.out = w_out;
  d.n_rows = m->n_rows;
  d.n_cols = m->n_cols;
  d.group = params->group;
  d.n_clusters = params->n_clusters;
  d.out_bf16 = out_dtype == ANY4_BF16 ? 1 : 0;
  return any4::launch_dequant(d, stream) == hipSuccess ? ANY4_OK : ANY4_ERR_HIP;
}

int any4_lut_gemv(const any4_matrix* m, const any4_params* params, const void* x, int32_t x_dtype,
                  int64_t n_tokens, float* y, hipStream_t stream) {
  if (!m || !params) return ANY4_ERR_INVALID_ARG;
  if (params->group < 2 || !is_pow2(params->group)) return ANY4_ERR_INVALID_ARG;
  if (!(params->n_clusters == 2 || params->n_clusters == 4 || params->n_clusters == 8 ||
        params->n_clusters == 16))
    return ANY4_ERR_INVALID_ARG;
  if (m->n_rows < 0 || m->n_cols < 2 || (m->n_cols & 1) || m->n_cols % params->group != 0)
    return ANY4_ERR_INVALID_ARG;
  if (x_dtype != ANY4_F32 && x_dtype != ANY4_BF16) return ANY4_ERR_INVALID_ARG;
  if (n_tokens < 1) return ANY4_ERR_INVALID_ARG;
  if (n_tokens > any4::kGemvMaxTokens || m->n_cols % 16 != 0 || params->group % 16 != 0)
    return ANY4_ERR_UNSUPPORTED;
  // rows index the grid and column offsets within a row are 32-bit in the kernel
  if (m->n_rows > INT32_MAX || m->n_cols > INT32_MAX) return ANY4_ERR_UNSUPPORTED;
  if (m->n_rows == 0) return ANY4_OK;
  if (!m->codes || !m->lut || !m->scale || !m->offset || !x || !y) return ANY4_ERR_INVALID_ARG;
  if ((reinterpret_cast<uintptr_t>(m->codes) & 7) != 0 || (reinterpret_cast<uintptr_t>(x) & 15) != 0)
    return ANY4_ERR_UNSUPPORTED;
  any4::GemvDesc d;
  std::memset(&d, 0, sizeof(d));
  d.codes = m->codes;
  d.lut = m->lut;
  d.scale = m->scale;
  d.offset = m->offset;
  d.x = x;
  d.y = y;
  d.n_tokens = n_tokens;
  d.n_rows = m->n_rows;
  d.n_cols = m->n_cols;
  d.group = params->group;
  d.n_clusters = params->n_clusters;
  d.x_bf16 = x_dtype == ANY4_BF16 ? 1 : 0;
  return any4::launch_gemv(d, stream) == hipSuccess ? ANY4_OK : ANY4_ERR_HIP;
}

}  // extern "C"
