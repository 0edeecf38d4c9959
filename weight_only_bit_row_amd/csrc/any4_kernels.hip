// gfx950 kernels of the any4 quantizer.
//
// One workgroup quantizes one weight row ("any4: Learned 4-bit Numeric Representation
// for LLMs", arXiv 2507.04610: Section 2.5.1 scaling, Section 4.1 E-step Eq. 18 and
// M-step Eq. 23, Appendix C.2 k-means++ initialisation, Section 2.4.1 storage).
// Rows are independent (Section 4.1 decouples the objective per output row), so the
// grid is one workgroup per row and no data crosses workgroups.
//
// Each lane owns E contiguous columns of the row; the row stays in VGPRs from the
// single HBM read to the single store of codes/LUT/scale/offset.
//
//   scale      group min/max in registers (shuffles for groups wider than a lane),
//              w_S = (w - beta) / alpha with IEEE division
//   seed       k-means++: sampling weights p_j updated in registers, exact integer
//              CDF (fp64 per-lane sums of floor(p_j 2^(40-e)), u64 scan across lanes),
//              Philox4x32-10 draw per (row, step)
//   Lloyd      per round: sort the <=16 centroids, merge equal values (lowest draw
//              index kept), compute the exact fp32 switch point between each pair of
//              sorted neighbours, then each element finds its cluster by a 4-level
//              binary search over the switch points (LDS, conflict-free: 15 entries),
//              and adds (a_j, a_j*w_S_j) in fp64 (the product is exact) into
//              lane-private LDS bins; bins are reduced per wave in a fixed order
//              (no global atomics)
//   emit       final assignment, nibble packing, fp16 LUT/scale/offset, fp64 objective
//
// All float code is compiled with -ffp-contract=off: every squared distance is
// fl(fl(x - c)^2), exactly as Eq. 18 is evaluated on the CPU side.
#include <hip/hip_runtime.h>
#include <hip/hip_fp16.h>
#include <stdint.h>

#include "any4_launch.h"

namespace any4 {
namespace {

constexpr int kWave = 64;
constexpr int kStatusNonfinite = 5;
constexpr float kAMax = 18446744073709551616.0f;  // 2^64: larger sample weights are rejected

// ---------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as
// 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies; the high halves are
// xor-ed with the other two words and the round key, the low halves become words 1
// and 3; the key is bumped by the golden-ratio and sqrt(3)-1 Weyl constants.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t lo0 = 0xD2511F53u * c[0], hi0 = __umulhi(0xD2511F53u, c[0]);
    const uint32_t lo1 = 0xCD9E8D57u * c[2], hi1 = __umulhi(0xCD9E8D57u, c[2]);
    const uint32_t n0 = hi1 ^ c[1] ^ k0;
    const uint32_t n2 = hi0 ^ c[3] ^ k1;
    c[0] = n0;
    c[1] = lo1;
    c[2] = n2;
    c[3] = lo0;
  }
}

// ---------------------------------------------------------------------------------
// Shared memory: a fixed header, then per-wave lane-private bins [nw][2][16][64] fp64.
struct Smem {
  float c[kMaxClusters];      // centroids in draw order
  float thr[kMaxClusters];    // switch points between sorted neighbours, +inf padded
  float sv[kMaxClusters];     // sorted distinct centroid values
  int sidx[kMaxClusters];     // lowest draw index holding each sorted value
  double red[2 * kMaxClusters];         // reduced bins: S0[16], S1[16]
  double wred[8][2 * kMaxClusters];     // per-wave partial bins
  float fred[2][8];                     // per-wave fp32 partials (double buffered)
  double dred[8];                       // per-wave fp64 partials
  unsigned long long ured[2][8];        // per-wave u64 partials (double buffered)
  unsigned long long u[kMaxClusters];   // Philox draw of each seeding step
  float stage_p[kWave];                 // sampling weights of the lane owning a pick
  float stage_x[kWave];                 // its scaled values
  int picks[kMaxClusters];
  unsigned long long owner_excl;
  float x0;                             // w_S of column 0
  float pick_c;
  int owner;
  int pick_j;
  int n_unique;
  int pad_[3];
};

constexpr size_t kSmemHdr = (sizeof(Smem) + 15) & ~size_t(15);
constexpr size_t kBinBytesPerWave = 2 * kMaxClusters * kWave * sizeof(double);  // 16 KiB

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ bool is_finite(float v) { return __builtin_isfinite(v); }

__device__ __forceinline__ uint16_t f16_bits(float v) {
  return __half_as_ushort(__float2half_rn(v));
}

__device__ __forceinline__ float uniform_f(float v) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// LDS traffic inside one wave needs no barrier, only a compiler/LDS ordering fence.
__device__ __forceinline__ void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  __builtin_amdgcn_wave_barrier();
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v = fmaxf(v, __shfl_xor(v, s));
  return v;
}
__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v = fminf(v, __shfl_xor(v, s));
  return v;
}
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int s = 32; s > 0; s >>= 1) v += __shfl_xor(v, s);
  return v;
}
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v, int lane) {
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    const unsigned long long t = __shfl_up(v, s);
    if (lane >= s) v += t;
  }
  return v;
}
__device__ __forceinline__ double wave_incl_scan_f64(double v, int lane) {
#pragma unroll
  for (int s = 1; s < kWave; s <<= 1) {
    const double t = __shfl_up(v, s);
    if (lane >= s) v += t;
  }
  return v;
}

// Pairwise rule between sorted neighbours L < R (values) with draw indices il, ir:
// R is chosen at x when its fp32 squared distance is smaller, or equal with the
// lower draw index (Eq. 18 with the lowest-index tie-break).
__device__ __forceinline__ bool right_wins(float x, float cl, int il, float cr, int ir) {
  float dl = x - cl;
  dl = dl * dl;
  float dr = x - cr;
  dr = dr * dr;
  return dr < dl || (dr == dl && ir < il);
}

// Smallest fp32 x in [cl, cr] (0 <= cl < cr) at which R wins.  The rule is monotone
// in x on that interval (left distance non-decreasing, right non-increasing under
// monotone rounding), so a bisection over the ordered bit patterns is exact.  The
// midpoint probe narrows the interval to a few ulps first.
__device__ float switch_point(float cl, int il, float cr, int ir) {
  uint32_t lo = __float_as_uint(cl), hi = __float_as_uint(cr);
  const float mid = cl + 0.5f * (cr - cl);
  const uint32_t mb = __float_as_uint(mid);
  if (mb >= lo + 2 && !right_wins(__uint_as_float(mb - 2), cl, il, cr, ir)) lo = mb - 1;
  if (mb + 2 <= hi && right_wins(__uint_as_float(mb + 2), cl, il, cr, ir)) hi = mb + 2;
  // invariant: every x below lo loses (or lo == cl), and hi wins (or hi == cr)
  for (int guard = 0; guard < 40 && lo < hi; ++guard) {
    const uint32_t m = lo + ((hi - lo) >> 1);
    if (right_wins(__uint_as_float(m), cl, il, cr, ir))
      hi = m;
    else
      lo = m + 1;
  }
  return __uint_as_float(hi);
}

// Wave 0 only: from S.c (k values), build the sorted distinct values, their lowest
// draw index, and the switch points S.thr[0..U-2] (+inf beyond).
__device__ void build_structure(Smem& S, int k, int lane) {
  const float inf = __builtin_huge_valf();
  float ct = (lane < k) ? S.c[lane] : inf;
  if (ct == 0.0f) ct = 0.0f;  // -0 -> +0 so that bit patterns order like values
  bool first = lane < k;
  for (int u = 0; u < k; ++u) {
    float cu = S.c[u];
    if (cu == 0.0f) cu = 0.0f;
    if (u < lane && cu == ct) first = false;
  }
  const unsigned long long fm = __ballot(first);
  int less = 0;
  for (int u = 0; u < k; ++u) {
    float cu = S.c[u];
    if (cu == 0.0f) cu = 0.0f;
    if (((fm >> u) & 1ull) && cu < ct) ++less;
  }
  const int U = __popcll(fm);
  if (first) {
    S.sv[less] = ct;
    S.sidx[less] = lane;
  }
  wave_lds_fence();
  if (lane < kMaxClusters) {
    float t = inf;
    if (lane + 1 < U) t = switch_point(S.sv[lane], S.sidx[lane], S.sv[lane + 1], S.sidx[lane + 1]);
    S.thr[lane] = t;
  }
  if (lane == 0) S.n_unique = U;
  wave_lds_fence();
}

// Cluster position (index into the sorted distinct values) of x: the number of
// switch points <= x, by a 4-level binary search over the 15 sorted switch points.
__device__ __forceinline__ int sorted_position(float x, float t7, const float* thr) {
  int pos = (x >= t7) ? 8 : 0;
  pos += (x >= thr[pos + 3]) ? 4 : 0;
  pos += (x >= thr[pos + 1]) ? 2 : 0;
  pos += (x >= thr[pos]) ? 1 : 0;
  return pos;
}

// ---------------------------------------------------------------------------------
// Row loading: lane owns columns [col0, col0 + E); missing columns read as 0.
template <int E>
__device__ __forceinline__ void load_row(const MatDesc& M, int64_t row, int K, int col0,
                                         float (&x)[E], float (&act)[E]) {
  const bool full = col0 + E <= K;
  if (M.dtype == 1) {
    const uint16_t* src = static_cast<const uint16_t*>(M.w) + row * (int64_t)K + col0;
    if (full && (K & 7) == 0 && ((reinterpret_cast<uintptr_t>(M.w) & 15) == 0)) {
#pragma unroll
      for (int v = 0; v < E / 8; ++v) {
        const uint4 d = reinterpret_cast<const uint4*>(src)[v];
        const uint32_t w4[4] = {d.x, d.y, d.z, d.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          x[8 * v + 2 * h] = bf16_bits_to_float(w4[h] & 0xFFFFu);
          x[8 * v + 2 * h + 1] = bf16_bits_to_float(w4[h] >> 16);
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < E; ++m) x[m] = (col0 + m < K) ? bf16_bits_to_float(src[m]) : 0.0f;
    }
  } else {
    const float* src = static_cast<const float*>(M.w) + row * (int64_t)K + col0;
    if (full && (K & 3) == 0 && ((reinterpret_cast<uintptr_t>(M.w) & 15) == 0)) {
#pragma unroll
      for (int v = 0; v < E / 4; ++v) {
        const float4 d = reinterpret_cast<const float4*>(src)[v];
        x[4 * v] = d.x;
        x[4 * v + 1] = d.y;
        x[4 * v + 2] = d.z;
        x[4 * v + 3] = d.w;
      }
    } else {
#pragma unroll
      for (int m = 0; m < E; ++m) x[m] = (col0 + m < K) ? src[m] : 0.0f;
    }
  }
  const float* asrc = M.act + col0;
  if (full && (K & 3) == 0 && ((reinterpret_cast<uintptr_t>(M.act) & 15) == 0)) {
#pragma unroll
    for (int v = 0; v < E / 4; ++v) {
      const float4 d = reinterpret_cast<const float4*>(asrc)[v];
      act[4 * v] = d.x;
      act[4 * v + 1] = d.y;
      act[4 * v + 2] = d.z;
      act[4 * v + 3] = d.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) act[m] = (col0 + m < K) ? asrc[m] : 0.0f;
  }
}

// Eq. 1-2 on one group held in registers [m0, m0+G), then the Eq. 23 sample weights.
// Writes alpha/beta of the group (fp32 for the scale stage, fp16 otherwise).
template <int MODE>
__device__ __forceinline__ void finish_group(float mn, float mx, float qr, float* x, float* act,
                                             int n, bool& bad, const MatDesc& M, int64_t row,
                                             int64_t gidx, int64_t n_groups, bool writer) {
  const float alpha = (mx - mn) / qr;
  const float beta = mn;
  if (!is_finite(alpha)) bad = true;
  for (int m = 0; m < n; ++m) {
    float ws = 0.0f;
    if (alpha > 0.0f) {
      const float diff = x[m] - beta;
      ws = diff / alpha;
    }
    const float a = alpha * act[m];
    if (!is_finite(a) || a > kAMax || !is_finite(a * ws)) bad = true;
    x[m] = ws;
    act[m] = a;
  }
  if (writer) {
    if (MODE == MODE_SCALE) {
      M.alpha_out[row * n_groups + gidx] = alpha;
      M.beta_out[row * n_groups + gidx] = beta;
    } else if (MODE == MODE_FULL) {
      M.scale[row * n_groups + gidx] = f16_bits(alpha);
      M.offset[row * n_groups + gidx] = f16_bits(beta);
    }
  }
}

// Groups no wider than a lane's E columns: G is a compile-time group size.
template <int E, int G, int MODE>
__device__ __forceinline__ void scale_narrow(float (&x)[E], float (&act)[E], float qr, int K,
                                             int col0, bool& bad, const MatDesc& M, int64_t row,
                                             int g) {
  const int64_t n_groups = K / g;
#pragma unroll
  for (int lg = 0; lg < E / G; ++lg) {
    const bool valid = col0 + lg * G < K;  // groups never straddle K (K % g == 0)
    float mn = x[lg * G], mx = x[lg * G];
#pragma unroll
    for (int m = 1; m < G; ++m) {
      mn = fminf(mn, x[lg * G + m]);
      mx = fmaxf(mx, x[lg * G + m]);
    }
    if (valid) {
      finish_group<MODE>(mn, mx, qr, &x[lg * G], &act[lg * G], G, bad, M, row,
                         (col0 + lg * G) / g, n_groups, true);
    } else {
#pragma unroll
      for (int m = 0; m < G; ++m) {
        x[lg * G + m] = 0.0f;
        act[lg * G + m] = 0.0f;
      }
    }
  }
}

// Groups spanning L = g / E lanes (L a power of two, lanes aligned to the group).
template <int E, int MODE>
__device__ __forceinline__ void scale_wide(float (&x)[E], float (&act)[E], float qr, int K,
                                           int col0, bool& bad, const MatDesc& M, int64_t row,
                                           int g, Smem& S, int lane, int wave, int nw) {
  const bool valid = col0 < K;
  float mn = x[0], mx = x[0];
#pragma unroll
  for (int m = 1; m < E; ++m) {
    mn = fminf(mn, x[m]);
    mx = fmaxf(mx, x[m]);
  }
  if (!valid) {
    mn = __builtin_huge_valf();
    mx = -__builtin_huge_valf();
  }
  const int L = g / E;
  if (L <= kWave) {
    for (int s = 1; s < L; s <<= 1) {
      mn = fminf(mn, __shfl_xor(mn, s));
      mx = fmaxf(mx, __shfl_xor(mx, s));
    }
  } else {  // group spans L / 64 whole waves (block-uniform branch)
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (lane == 0) {
      S.fred[0][wave] = mn;
      S.fred[1][wave] = mx;
    }
    __syncthreads();
    const int wpg = L / kWave;
    const int w0 = (wave / wpg) * wpg;
    for (int w = w0; w < w0 + wpg && w < nw; ++w) {
      mn = fminf(mn, S.fred[0][w]);
      mx = fmaxf(mx, S.fred[1][w]);
    }
    __syncthreads();
  }
  if (valid) {
    finish_group<MODE>(mn, mx, qr, x, act, E, bad, M, row, col0 / g, K / g, (col0 % g) == 0);
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) {
      x[m] = 0.0f;
      act[m] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------------
// E-step + M-step over the lane's elements: position by binary search, then the two
// Eq. 23 sums into lane-private fp64 bins (address pos*64 + lane: conflict-free).
// (double)a * (double)w_S is exact, so only the order of the fp64 additions differs
// from a sequential sum.
// The resident row is re-declared opaque on every round: otherwise the compiler
// hoists the loop-invariant fp64 conversions out of the Lloyd loop and holds 4E
// extra registers.
template <int E>
__device__ __forceinline__ void pin_row(float (&x)[E], float (&a)[E]) {
#pragma unroll
  for (int m = 0; m < E; ++m) asm volatile("" : "+v"(x[m]), "+v"(a[m]));
}

template <int E>
__device__ __forceinline__ void em_pass(float (&x)[E], float (&a)[E], const Smem& S,
                                        double* bins, int lane) {
  pin_row<E>(x, a);
  const float t7 = uniform_f(S.thr[7]);
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int pos = sorted_position(x[m], t7, S.thr);
    double* b = bins + pos * kWave + lane;
    const double ad = static_cast<double>(a[m]);
    atomicAdd(b, ad);
    atomicAdd(b + kMaxClusters * kWave, ad * static_cast<double>(x[m]));
  }
}

// Reduce this wave's bins into 32 slot sums (S0[0..15], S1[0..15]) and clear them.
// Lane l sums slot l>>1 over 32 lanes' partials in a fixed rotated order (rotation
// keeps the 16-byte reads of 8 consecutive lanes on distinct banks).
__device__ __forceinline__ double reduce_bins(double* bins, int lane) {
  const int slot = lane >> 1, half = lane & 1;
  double2* src = reinterpret_cast<double2*>(bins + slot * kWave + half * 32);
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int j = (i + lane) & 15;
    const double2 v = src[j];
    s += v.x;
    s += v.y;
    src[j] = make_double2(0.0, 0.0);
  }
  const double other = __shfl_xor(s, 1);
  return half ? other + s : s + other;  // same order in both lanes of the pair
}

__device__ __forceinline__ void zero_bins(double* bins, int lane) {
  double2* dst = reinterpret_cast<double2*>(bins + lane * 32);
#pragma unroll
  for (int i = 0; i < 16; ++i) dst[i] = make_double2(0.0, 0.0);
}

// All-waves step: bins -> S.red (block-wide slot sums).
__device__ __forceinline__ void block_reduce_bins(Smem& S, double* bins, int lane, int wave,
                                                  int nw) {
  const double s = reduce_bins(bins, lane);
  if (nw == 1) {
    if ((lane & 1) == 0) S.red[lane >> 1] = s;
    __syncthreads();
  } else {
    if ((lane & 1) == 0) S.wred[wave][lane >> 1] = s;
    __syncthreads();
    if (wave == 0 && lane < 2 * kMaxClusters) {
      double t = S.wred[0][lane];
      for (int w = 1; w < nw; ++w) t += S.wred[w][lane];
      S.red[lane] = t;
    }
    __syncthreads();
  }
}

// Wave 0: Eq. 23 update, the fp64 ratio rounded to fp32; an empty cluster (zero
// weight) keeps its value.
__device__ __forceinline__ void update_centroids(Smem& S, int lane, int wave) {
  if (wave == 0 && lane < S.n_unique) {
    const double s0 = S.red[lane], s1 = S.red[kMaxClusters + lane];
    if (s0 > 0.0) S.c[S.sidx[lane]] = static_cast<float>(s1 / s0);
  }
}

__device__ __forceinline__ float block_max(float v, Smem& S, int lane, int wave, int nw,
                                           int parity) {
  v = wave_max(v);
  if (nw == 1) return v;
  if (lane == 0) S.fred[parity][wave] = v;
  __syncthreads();
  float r = S.fred[parity][0];
  for (int w = 1; w < nw; ++w) r = fmaxf(r, S.fred[parity][w]);
  return r;
}

__device__ __forceinline__ double block_sum_f64(double v, Smem& S, int lane, int wave, int nw) {
  v = wave_sum_f64(v);
  if (nw == 1) return v;
  __syncthreads();
  if (lane == 0) S.dred[wave] = v;
  __syncthreads();
  double r = S.dred[0];
  for (int w = 1; w < nw; ++w) r += S.dred[w];
  return r;
}

// ---------------------------------------------------------------------------------
template <int E, int NWMAX, int MODE>
__global__ __launch_bounds__(kWave* NWMAX) void any4_rows_kernel(const LaunchArgs args) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  const int nw = (NWMAX == 1) ? 1 : args.nw;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid >> 6;

  const int64_t b = blockIdx.x;
  int mi = 0;
#pragma unroll
  for (int i = 1; i < kMaxMats; ++i)
    if (i < args.n_mats && b >= args.row_start[i]) mi = i;
  const MatDesc& M = args.m[mi];
  const int64_t row = b - args.row_start[mi];
  const int K = static_cast<int>(M.n_cols);
  const int g = args.group;
  const int k = args.n_clusters;
  const float qr = static_cast<float>(k - 1);
  const int col0 = tid * E;

  float xv[E], av[E];
  load_row<E>(M, row, K, col0, xv, av);

  bool bad = false;
#pragma unroll
  for (int m = 0; m < E; ++m) {
    if (col0 + m < K) {
      if (!is_finite(xv[m])) bad = true;
      if (!(av[m] >= 0.0f) || !is_finite(av[m])) bad = true;
    }
  }

  // ---- Eq. 1-2 scaling and Eq. 23 sample weights
  if (g >= E) {
    scale_wide<E, MODE>(xv, av, qr, K, col0, bad, M, row, g, S, lane, wave, nw);
  } else {
    switch (g) {
      case 2: scale_narrow<E, 2, MODE>(xv, av, qr, K, col0, bad, M, row, g); break;
      case 4: scale_narrow<E, 4, MODE>(xv, av, qr, K, col0, bad, M, row, g); break;
      case 8: if constexpr (E > 8) scale_narrow<E, 8, MODE>(xv, av, qr, K, col0, bad, M, row, g); break;
      case 16: if constexpr (E > 16) scale_narrow<E, 16, MODE>(xv, av, qr, K, col0, bad, M, row, g); break;
      case 32: if constexpr (E > 32) scale_narrow<E, 32, MODE>(xv, av, qr, K, col0, bad, M, row, g); break;
      default: break;
    }
  }

  if (MODE == MODE_SCALE) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
      if (col0 + m < K) {
        M.ws_out[row * K + col0 + m] = xv[m];
        M.a_out[row * K + col0 + m] = av[m];
      }
    }
    return;
  }

  if (tid == 0) S.x0 = xv[0];
  const bool row_bad = __syncthreads_or(bad);
  if (row_bad) {
    if (MODE == MODE_FULL) {
      for (int m = 0; m < E; m += 2)
        if (col0 + m < K) M.codes[row * (K / 2) + (col0 + m) / 2] = 0;
      if (tid < k) M.lut[row * k + tid] = 0;
      // the lanes that wrote alpha/beta of a group overwrite them
      for (int c = col0; c < col0 + E && c < K; c += (g < E ? g : E)) {
        if (c % g == 0) {
          M.scale[row * (K / g) + c / g] = 0;
          M.offset[row * (K / g) + c / g] = 0;
        }
      }
      if (tid == 0) {
        if (M.objective) M.objective[row] = __builtin_nan("");
        if (args.status) atomicOr(args.status, (uint32_t)kStatusNonfinite);
      }
    }
    return;
  }

  // ---- k-means++ seeding (or the given centroids for a single Lloyd round)
  if (MODE == MODE_STEP) {
    if (tid < k) S.c[tid] = M.c_in[row * k + tid];
    __syncthreads();
  } else {
    if (tid < k) {
      const uint64_t rid = static_cast<uint64_t>(M.row_offset + row);
      uint32_t c[4] = {static_cast<uint32_t>(rid), static_cast<uint32_t>(tid),
                       static_cast<uint32_t>(M.matrix_index), static_cast<uint32_t>(rid >> 32)};
      philox4x32_10(c, static_cast<uint32_t>(args.seed), static_cast<uint32_t>(args.seed >> 32));
      S.u[tid] = (static_cast<unsigned long long>(c[1]) << 32) | c[0];
    }
    float pv[E];
#pragma unroll
    for (int m = 0; m < E; ++m) pv[m] = av[m];
    __syncthreads();
    for (int t = 0; t < k; ++t) {
      float lmax = 0.0f;
#pragma unroll
      for (int m = 0; m < E; ++m) lmax = fmaxf(lmax, pv[m]);
      const float pmax = block_max(lmax, S, lane, wave, nw, t & 1);
      float ct;
      int pick;
      if (pmax == 0.0f) {
        ct = (t == 0) ? S.x0 : S.c[0];
        pick = -1;
      } else {
        int e2;
        frexpf(pmax, &e2);
        const double sc = ldexp(1.0, 40 - (e2 - 1));  // 2^(40 - floor(log2 pmax))
        double lsum = 0.0;
#pragma unroll
        for (int m = 0; m < E; ++m) lsum += floor(static_cast<double>(pv[m]) * sc);
        const unsigned long long ls = static_cast<unsigned long long>(lsum);
        const unsigned long long incl = wave_incl_scan_u64(ls, lane);
        unsigned long long woff = 0, Q = __shfl(incl, kWave - 1);
        if (nw > 1) {
          if (lane == kWave - 1) S.ured[t & 1][wave] = incl;
          __syncthreads();
          Q = 0;
          for (int w = 0; w < nw; ++w) {
            const unsigned long long v = S.ured[t & 1][w];
            if (w < wave) woff += v;
            Q += v;
          }
        }
        const unsigned long long excl = woff + incl - ls;
        const unsigned long long r = __umul64hi(S.u[t], Q);
        const bool own = ls > 0 && excl <= r && r - excl < ls;
        if (own) {
          S.owner = tid;
          S.owner_excl = excl;
#pragma unroll
          for (int m = 0; m < E; ++m) {
            S.stage_p[m] = pv[m];
            S.stage_x[m] = xv[m];
          }
        }
        __syncthreads();
        if (wave == 0) {
          const unsigned long long oex = S.owner_excl;
          const double q = (lane < E) ? floor(static_cast<double>(S.stage_p[lane]) * sc) : 0.0;
          const double qi = wave_incl_scan_f64(q, lane);
          const bool hit = lane < E && oex + static_cast<unsigned long long>(qi) > r;
          const unsigned long long bal = __ballot(hit);
          int ms = __ffsll(static_cast<long long>(bal)) - 1;
          if (ms < 0) ms = E - 1;  // unreachable: the owner's prefix always crosses r
          if (lane == 0) {
            S.pick_c = S.stage_x[ms];
            S.pick_j = S.owner * E + ms;
          }
        }
        __syncthreads();
        ct = S.pick_c;
        pick = S.pick_j;
      }
      if (tid == 0) {
        S.c[t] = ct;
        S.picks[t] = pick;
      }
      // sampling weights for the next draw: a_j * min_t fl((w_S_j - c_t)^2)
#pragma unroll
      for (int m = 0; m < E; ++m) {
        float d = xv[m] - ct;
        d = d * d;
        const float pd = av[m] * d;
        pv[m] = (t == 0) ? pd : fminf(pv[m], pd);
      }
    }
    __syncthreads();
    if (MODE == MODE_SEED) {
      if (tid < k) {
        M.c_out[row * k + tid] = S.c[tid];
        M.picks_out[row * k + tid] = S.picks[tid];
      }
      return;
    }
    if (M.picks_out && tid < k) M.picks_out[row * k + tid] = S.picks[tid];
  }

  // ---- Lloyd rounds
  double* bins = reinterpret_cast<double*>(smem_raw + kSmemHdr) + wave * (2 * kMaxClusters * kWave);
  zero_bins(bins, lane);
  const int rounds = (MODE == MODE_STEP) ? 1 : args.iters;
  for (int it = 0; it < rounds; ++it) {
    if (wave == 0) build_structure(S, k, lane);
    __syncthreads();
    if (MODE == MODE_STEP) {
      // E-step with its assignment and objective at c_in, then the same bin sums
      const float t7 = uniform_f(S.thr[7]);
      double J = 0.0;
#pragma unroll
      for (int m = 0; m < E; ++m) {
        const int pos = sorted_position(xv[m], t7, S.thr);
        double* bp = bins + pos * kWave + lane;
        const double ad = static_cast<double>(av[m]);
        atomicAdd(bp, ad);
        atomicAdd(bp + kMaxClusters * kWave, ad * static_cast<double>(xv[m]));
        if (col0 + m < K) {
          M.assign_out[row * K + col0 + m] = static_cast<uint8_t>(S.sidx[pos]);
          const double d = static_cast<double>(xv[m]) - static_cast<double>(S.sv[pos]);
          J += static_cast<double>(av[m]) * d * d;
        }
      }
      J = block_sum_f64(J, S, lane, wave, nw);
      if (tid == 0 && M.objective) M.objective[row] = J;
    } else {
      if (col0 < K) em_pass<E>(xv, av, S, bins, lane);
    }
    __syncthreads();
    block_reduce_bins(S, bins, lane, wave, nw);
    update_centroids(S, lane, wave);
    __syncthreads();
  }
  if (MODE == MODE_STEP) {
    if (tid < k) M.c_out[row * k + tid] = S.c[tid];
    return;
  }

  // ---- final E-step, objective and emission
  if (wave == 0) build_structure(S, k, lane);
  __syncthreads();
  const float t7 = uniform_f(S.thr[7]);
  double J = 0.0;
  uint32_t packed[E / 8];
#pragma unroll
  for (int v = 0; v < E / 8; ++v) packed[v] = 0;
#pragma unroll
  for (int m = 0; m < E; ++m) {
    const int pos = sorted_position(xv[m], t7, S.thr);
    const uint32_t q = static_cast<uint32_t>(S.sidx[pos]);
    packed[m / 8] |= q << (4 * (m % 8));
    const double d = static_cast<double>(xv[m]) - static_cast<double>(S.sv[pos]);
    J += static_cast<double>(av[m]) * d * d;
  }
  if (col0 < K) {
    uint8_t* dst = M.codes + row * (K / 2) + col0 / 2;
    const bool vec = (col0 + E <= K) && ((K / 2) % 16 == 0) &&
                     ((reinterpret_cast<uintptr_t>(M.codes) & 15) == 0);
    if (vec && E >= 32) {
#pragma unroll
      for (int v = 0; v < E / 32; ++v)
        reinterpret_cast<uint4*>(dst)[v] =
            make_uint4(packed[4 * v], packed[4 * v + 1], packed[4 * v + 2], packed[4 * v + 3]);
    } else {
#pragma unroll
      for (int m = 0; m < E; m += 2)
        if (col0 + m < K) dst[m / 2] = static_cast<uint8_t>(packed[m / 8] >> (4 * (m % 8)));
    }
  }
  J = block_sum_f64(J, S, lane, wave, nw);
  if (tid == 0 && M.objective) M.objective[row] = J;
  if (tid < k) {
    M.lut[row * k + tid] = f16_bits(S.c[tid]);
    if (M.c_out) M.c_out[row * k + tid] = S.c[tid];
  }
}

__global__ void clear_status_kernel(uint32_t* status) {
  if (threadIdx.x == 0) *status = 0u;
}

// Emission only, from given assignments/centroids/scales: one thread per packed byte.
__global__ void pack_kernel(MatDesc M, int group, int k, const uint8_t* assign, const float* c,
                            const float* alpha, const float* beta) {
  const int64_t K = M.n_cols;
  const int64_t n_bytes = M.n_rows * (K / 2);
  const int64_t n_groups = K / group;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n_bytes;
       i += (int64_t)gridDim.x * blockDim.x) {
    M.codes[i] = static_cast<uint8_t>((assign[2 * i] & 0xF) | ((assign[2 * i + 1] & 0xF) << 4));
  }
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < M.n_rows * k;
       i += (int64_t)gridDim.x * blockDim.x)
    M.lut[i] = f16_bits(c[i]);
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < M.n_rows * n_groups;
       i += (int64_t)gridDim.x * blockDim.x) {
    M.scale[i] = f16_bits(alpha[i]);
    M.offset[i] = f16_bits(beta[i]);
  }
}

template <int E, int NWMAX>
hipError_t launch_mode(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  const int nw = (NWMAX == 1) ? 1 : args.nw;
  const size_t smem = kSmemHdr + ((mode == MODE_FULL || mode == MODE_STEP)
                                      ? static_cast<size_t>(nw) * kBinBytesPerWave
                                      : 0);
  const dim3 grid(static_cast<unsigned>(n_blocks));
  const dim3 block(kWave * nw);
  switch (mode) {
    case MODE_FULL:
      hipLaunchKernelGGL((any4_rows_kernel<E, NWMAX, MODE_FULL>), grid, block, smem, stream, args);
      break;
    case MODE_SCALE:
      hipLaunchKernelGGL((any4_rows_kernel<E, NWMAX, MODE_SCALE>), grid, block, smem, stream, args);
      break;
    case MODE_SEED:
      hipLaunchKernelGGL((any4_rows_kernel<E, NWMAX, MODE_SEED>), grid, block, smem, stream, args);
      break;
    case MODE_STEP:
      hipLaunchKernelGGL((any4_rows_kernel<E, NWMAX, MODE_STEP>), grid, block, smem, stream, args);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

RowConfig choose_config(int64_t K) {
  if (K <= 512) return {8, 1};
  if (K <= 1024) return {16, 1};
  if (K <= 2048) return {32, 1};
  if (K <= 4096) return {64, 1};
  // several waves per row: least padding, then the larger E
  const int64_t nw64 = (K + 4095) / 4096, nw32 = (K + 2047) / 2048;
  const int64_t pad64 = nw64 * 4096 - K, pad32 = nw32 * 2048 - K;
  if (nw32 <= 8 && pad32 < pad64) return {32, static_cast<int>(nw32)};
  return {64, static_cast<int>(nw64)};
}

hipError_t launch_rows(const LaunchArgs& args, RowConfig cfg, int mode, int64_t n_blocks,
                       hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  if (cfg.nw == 1) {
    switch (cfg.e) {
      case 8: return launch_mode<8, 1>(args, mode, n_blocks, stream);
      case 16: return launch_mode<16, 1>(args, mode, n_blocks, stream);
      case 32: return launch_mode<32, 1>(args, mode, n_blocks, stream);
      case 64: return launch_mode<64, 1>(args, mode, n_blocks, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (cfg.e) {
    case 32: return launch_mode<32, 8>(args, mode, n_blocks, stream);
    case 64: return launch_mode<64, 8>(args, mode, n_blocks, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_clear_status(uint32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(clear_status_kernel, dim3(1), dim3(64), 0, stream, status);
  return hipGetLastError();
}

hipError_t launch_pack(const MatDesc& m, int group, int n_clusters, const uint8_t* assign,
                       const float* c, const float* alpha, const float* beta,
                       hipStream_t stream) {
  const int64_t n = m.n_rows * (m.n_cols / 2);
  int64_t blocks = (n + 255) / 256;
  if (blocks < 1) blocks = 1;
  if (blocks > 65536) blocks = 65536;
  hipLaunchKernelGGL(pack_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream, m,
                     group, n_clusters, assign, c, alpha, beta);
  return hipGetLastError();
}

}  // namespace any4
