// Drives every entry point of include/any4.h through valid and invalid arguments on the
// host (the kernel launchers are stand-ins, see abi_stubs.cpp), under AddressSanitizer
// and UndefinedBehaviorSanitizer.  Exits 0 and prints "ok" when every status code is the
// documented one.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "any4.h"

extern int g_row_launches;
extern int64_t g_rows_launched;

static int g_failures = 0;
#define EXPECT(expr, want)                                                            \
  do {                                                                                \
    const int got_ = (expr);                                                          \
    if (got_ != (want)) {                                                             \
      std::fprintf(stderr, "line %d: %s -> %d, want %d\n", __LINE__, #expr, got_, want); \
      ++g_failures;                                                                   \
    }                                                                                 \
  } while (0)

static void* P(uintptr_t v) { return reinterpret_cast<void*>(v); }

static any4_matrix mat(int64_t n, int64_t k, int32_t dtype = ANY4_BF16) {
  any4_matrix m{};
  m.w = P(0x1000);
  m.w_dtype = dtype;
  m.n_rows = n;
  m.n_cols = k;
  m.act_absmean = static_cast<const float*>(P(0x2000));
  m.codes = static_cast<uint8_t*>(P(0x3000));
  m.lut = static_cast<uint16_t*>(P(0x4000));
  m.scale = static_cast<uint16_t*>(P(0x5000));
  m.offset = static_cast<uint16_t*>(P(0x6000));
  return m;
}

int main() {
  const any4_params p{128, 16, 20, 0, 0};
  any4_params bad_group = p;
  bad_group.group = 96;
  size_t bytes = 0;

  // workspace query and validation
  any4_matrix m = mat(4, 512);
  EXPECT(any4_workspace_bytes(&m, 1, &p, &bytes), ANY4_OK);
  EXPECT(any4_workspace_bytes(&m, 1, &bad_group, &bytes), ANY4_ERR_INVALID_ARG);
  EXPECT(any4_workspace_bytes(&m, 1, nullptr, &bytes), ANY4_ERR_INVALID_ARG);
  EXPECT(any4_workspace_bytes(nullptr, 1, &p, &bytes), ANY4_ERR_INVALID_ARG);
  EXPECT(any4_workspace_bytes(&m, 1, &p, nullptr), ANY4_ERR_INVALID_ARG);
  any4_matrix odd = mat(4, 513);
  EXPECT(any4_workspace_bytes(&odd, 1, &p, &bytes), ANY4_ERR_INVALID_ARG);
  any4_matrix longrow = mat(4, 65536);
  EXPECT(any4_workspace_bytes(&longrow, 1, &p, &bytes), ANY4_ERR_UNSUPPORTED);
  any4_params var = p;
  var.variant = 1 << 6;
  EXPECT(any4_workspace_bytes(&m, 1, &var, &bytes), ANY4_ERR_INVALID_ARG);
  var.variant = ANY4_ALL_ROUNDS;
  EXPECT(any4_workspace_bytes(&m, 1, &var, &bytes), ANY4_OK);

  // a mixed batch: 12 matrices over every row geometry, with and without restarts
  std::vector<any4_matrix> batch;
  const int64_t cols[] = {2, 96, 512, 1000, 1024, 2048, 4096, 8192, 14336, 16384, 28672, 32768};
  int64_t total_rows = 0;
  for (int i = 0; i < 12; ++i) {
    batch.push_back(mat(3 + i, cols[i]));
    batch.back().matrix_index = i;
    total_rows += 3 + i;
  }
  any4_params q2 = p;
  q2.group = 2;
  for (int restarts = 1; restarts <= 3; restarts += 2) {
    any4_params q = q2;
    q.variant = (restarts - 1) << 8;
    EXPECT(any4_workspace_bytes(batch.data(), 12, &q, &bytes), ANY4_OK);
    std::vector<unsigned char> ws(bytes);  // host memory: the stand-ins only carve it
    g_row_launches = 0;
    g_rows_launched = 0;
    EXPECT(any4_quantize(batch.data(), 12, &q, ws.data(), ws.size(), nullptr), ANY4_OK);
    if (g_rows_launched != total_rows * restarts) {
      std::fprintf(stderr, "rows launched %lld, want %lld\n", (long long)g_rows_launched,
                   (long long)(total_rows * restarts));
      ++g_failures;
    }
    EXPECT(any4_quantize(batch.data(), 12, &q, ws.data(), ws.size() - 1, nullptr), ANY4_ERR_WORKSPACE);
    std::vector<float*> cf(12, static_cast<float*>(P(0x8000)));
    std::vector<int32_t*> pk(12, nullptr);
    EXPECT(any4_stage_quantize_batch(batch.data(), 12, &q, cf.data(), pk.data(), ws.data(), ws.size(),
                                     nullptr), ANY4_OK);
    EXPECT(any4_stage_quantize_batch(batch.data(), 12, &q, nullptr, nullptr, ws.data(), ws.size(),
                                     nullptr), ANY4_OK);
  }
  // zero-row matrices need no pointers
  any4_matrix empty{};
  empty.n_cols = 256;
  empty.w_dtype = ANY4_F32;
  unsigned char ws256[256];
  EXPECT(any4_quantize(&empty, 1, &p, ws256, sizeof(ws256), nullptr), ANY4_OK);
  EXPECT(any4_quantize(&m, 0, &p, ws256, sizeof(ws256), nullptr), ANY4_OK);
  EXPECT(any4_quantize(&m, -1, &p, ws256, sizeof(ws256), nullptr), ANY4_ERR_INVALID_ARG);

  // the entry point that allocates nothing
  EXPECT(any4_quantize_noalloc(batch.data(), 12, &q2, nullptr, nullptr), ANY4_OK);
  EXPECT(any4_quantize_noalloc(batch.data(), 12, &q2, static_cast<uint32_t*>(P(0x9000)), nullptr), ANY4_OK);
  std::vector<any4_matrix> many(ANY4_NOALLOC_MAX_MATRICES + 1, mat(1, 64));
  any4_params g64 = p;
  g64.group = 64;
  EXPECT(any4_quantize_noalloc(many.data(), ANY4_NOALLOC_MAX_MATRICES, &g64, nullptr, nullptr), ANY4_OK);
  EXPECT(any4_quantize_noalloc(many.data(), ANY4_NOALLOC_MAX_MATRICES + 1, &g64, nullptr, nullptr),
         ANY4_ERR_UNSUPPORTED);
  any4_matrix big = mat(20000, 4096);
  any4_params r2 = p;
  r2.variant = 1 << 8;
  EXPECT(any4_quantize_noalloc(&big, 1, &r2, nullptr, nullptr), ANY4_ERR_WORKSPACE);

  // stage entry points
  float* f = static_cast<float*>(P(0xA000));
  EXPECT(any4_stage_scale(&m, &p, f, f, f, f, nullptr), ANY4_OK);
  EXPECT(any4_stage_scale(&m, &p, nullptr, f, f, f, nullptr), ANY4_ERR_INVALID_ARG);
  EXPECT(any4_stage_seed(&m, &p, f, static_cast<int32_t*>(P(0xB000)), nullptr), ANY4_OK);
  EXPECT(any4_stage_seed(&m, &p, nullptr, nullptr, nullptr), ANY4_ERR_INVALID_ARG);
  EXPECT(any4_stage_lloyd_step(&m, &p, f, static_cast<uint8_t*>(P(0xC000)), f, nullptr, nullptr), ANY4_OK);
  EXPECT(any4_stage_lloyd_sorted(&m, &p, f, f, f, f, nullptr, 0, nullptr), ANY4_OK);
  any4_matrix m17k = mat(2, 16386);   // past 16384 columns: two halves and a workspace
  any4_params g8 = p;
  g8.group = 8;
  EXPECT(any4_stage_lloyd_sorted_workspace_bytes(2, 16386, &bytes), ANY4_OK);
  EXPECT(bytes == 2u * 3u * 16384u * 4u ? 1 : 0, 1);
  EXPECT(any4_stage_lloyd_sorted(&m17k, &g8, f, f, f, f, nullptr, 0, nullptr), ANY4_ERR_WORKSPACE);
  EXPECT(any4_stage_lloyd_sorted(&m17k, &g8, f, f, f, f, P(0xD000), bytes - 1, nullptr), ANY4_ERR_WORKSPACE);
  EXPECT(any4_stage_lloyd_sorted(&m17k, &g8, f, f, f, f, P(0xD000), bytes, nullptr), ANY4_OK);
  any4_matrix m33k = mat(2, 32770);   // past 32768 columns
  EXPECT(any4_stage_lloyd_sorted(&m33k, &g8, f, f, f, f, P(0xD000), bytes, nullptr), ANY4_ERR_UNSUPPORTED);
  EXPECT(any4_stage_lloyd_sorted_workspace_bytes(2, 32770, &bytes), ANY4_ERR_UNSUPPORTED);
  EXPECT(any4_stage_lloyd_sorted_workspace_bytes(2, 4096, &bytes), ANY4_OK);
  EXPECT(bytes == 0 ? 1 : 0, 1);
  EXPECT(any4_stage_pack(&m, &p, static_cast<uint8_t*>(P(0xC000)), f, f, f, nullptr), ANY4_OK);
  EXPECT(any4_stage_full(&m, &p, f, nullptr, ws256, sizeof(ws256), nullptr), ANY4_OK);
  EXPECT(any4_stage_full(&m, &p, f, nullptr, nullptr, 0, nullptr), ANY4_ERR_WORKSPACE);

  // bookends
  EXPECT(any4_act_absmean_workspace_bytes(1000, 4096, &bytes), ANY4_OK);
  std::vector<unsigned char> aws(bytes);
  EXPECT(any4_act_absmean(P(0x1000), ANY4_BF16, 1000, 4096, f, aws.data(), aws.size(), nullptr), ANY4_OK);
  EXPECT(any4_act_absmean(P(0x1000), ANY4_BF16, 1000, 4096, f, aws.data(), aws.size() - 1, nullptr),
         ANY4_ERR_WORKSPACE);
  EXPECT(any4_act_absmean(P(0x1000), 3, 1000, 4096, f, aws.data(), aws.size(), nullptr), ANY4_ERR_INVALID_ARG);
  EXPECT(any4_dequantize(&m, &p, f, ANY4_BF16, nullptr), ANY4_OK);
  EXPECT(any4_dequantize(&m, &p, f, 7, nullptr), ANY4_ERR_INVALID_ARG);
  EXPECT(any4_lut_gemv(&m, &p, P(0x1000), ANY4_BF16, 8, f, nullptr), ANY4_OK);
  EXPECT(any4_lut_gemv(&m, &p, P(0x1000), ANY4_BF16, 9, f, nullptr), ANY4_ERR_UNSUPPORTED);
  EXPECT(any4_lut_gemv(&m, &p, P(0x1004), ANY4_BF16, 1, f, nullptr), ANY4_ERR_UNSUPPORTED);

  // geometry, status strings, device status
  int32_t e = 0, nw = 0;
  EXPECT(any4_launch_geometry(28672, &e, &nw), ANY4_OK);
  if (e != 32 || nw != 14) ++g_failures;
  EXPECT(any4_launch_geometry(1, &e, &nw), ANY4_ERR_INVALID_ARG);
  for (int s = -1; s < 8; ++s)
    if (!any4_status_string(s)) ++g_failures;
  EXPECT(any4_read_device_status(ws256, nullptr), ANY4_OK);
  EXPECT(any4_read_device_status(nullptr, nullptr), ANY4_ERR_WORKSPACE);

  if (g_failures) {
    std::fprintf(stderr, "%d failures\n", g_failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
