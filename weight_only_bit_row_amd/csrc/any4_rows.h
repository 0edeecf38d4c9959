// Device code of the any4 row kernel, shared by the translation units that
// instantiate it (one per row geometry, so that they compile in parallel) and by
// the sorted-row stage in any4_kernels.hip.  Everything here has internal linkage.
#pragma once
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
//   scale      group min/max in registers (DPP moves for groups wider than a lane),
//              w_S = (w - beta) / alpha correctly rounded (IEEE division, or one fp64
//              reciprocal per group where a lane holds one group)
//   seed       k-means++: sampling weights p_j held scaled by 2^(40-e), in registers
//              (in the bin area for rows of 5-16 waves), exact integer CDF (fp64 per-lane
//              sums of floor(p_j 2^(40-e)), u64 scan across lanes), one Philox4x32-10
//              draw per (row, step); the serial chain of each draw at raised priority
//   Lloyd      per round: sort the <=16 centroids, merge equal values (lowest draw
//              index kept), compute the exact fp32 switch point between each pair of
//              sorted neighbours, and tabulate them over 2k fixed cells, each half a
//              scaled unit wide (per cell, 8 bytes: cluster position at the cell start
//              and the switch point inside it).  Each element's cell is fixed for the whole
//              row, so its E-step is one 8-byte LDS read and one compare; a round whose
//              table would need a second switch point in one cell uses a 4-level
//              binary search over all switch points instead (same result).  The
//              element then adds (a_j, a_j*w_S_j) in fp64 (the product is exact) into
//              lane-private LDS bins, reduced in a fixed order (one-wave rows); rows of
//              2-16 waves add the same terms in 64-bit fixed point (exact integer sums)
//              into one set of bins for the whole row (no global atomics)
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
// greedy k-means++: candidates per draw, 2 + floor(ln k) (2, 3, 4, 4 for k = 2, 4, 8, 16)
constexpr int kMaxTrials = 4;
__device__ __forceinline__ int greedy_trials(int k) { return k <= 2 ? 2 : (k == 4 ? 3 : 4); }

constexpr int kMaxWaves = 16;  // waves per row: 1024-lane workgroups

struct Smem {
  float c[kMaxClusters];      // centroids in draw order
  float thr[kMaxClusters + 4];       // switch points between sorted neighbours, +inf padded
  uint32_t tcell[kMaxClusters + 4];  // cell of each switch point, kMaxCells beyond the last
  float sv[kMaxClusters];     // sorted distinct centroid values
  int sidx[kMaxClusters];     // lowest draw index holding each sorted value
  union {
    double wred[kMaxWaves][2 * kMaxClusters];   // per-wave partial bins (Lloyd rounds)
    struct {                            // greedy k-means++ (seeding)
      unsigned long long u[kMaxTrials - 1][kMaxClusters];  // draws of candidates 1..
      unsigned long long pot[kMaxWaves][kMaxTrials];               // per-wave candidate potentials
      float cand_c[kMaxTrials];
      int cand_j[kMaxTrials];
    } gk;
  };
  float fred[2][kMaxWaves];                     // per-wave fp32 partials (double buffered)
  double dred[kMaxWaves];                       // per-wave fp64 partials
  alignas(16) unsigned long long ured[2][kMaxWaves];  // per-wave u64 partials (double buffered)
  unsigned long long u[kMaxClusters];   // Philox draw of each seeding step
  int picks[kMaxClusters];
  float x0;                             // w_S of column 0
  float pick_c;
  int pick_j;
  int n_unique;
  int use_table;                        // this round's cell table is complete
  int bad[kMaxWaves];                           // per-wave vote: the row holds a bad value
  float rstat[3][kMaxWaves];                    // per-wave max a, min w_S, max w_S
  int done;                                     // the centroids reached a fixed point
  int pad_[1];
};

constexpr size_t kSmemHdr = (sizeof(Smem) + 15) & ~size_t(15);
constexpr int kCellsPerUnit = 2;                           // cell width 1/2 of a scaled unit
constexpr int kMaxCells = kCellsPerUnit * kMaxClusters;    // cells cover [0, n_clusters)
constexpr int kCellBytes = 8;                              // {T, position} per cell
constexpr size_t kTableBytes = kMaxCells * kCellBytes;
// Each element keeps the byte offset of its table cell (cell * 8 < 256) in an 8-bit
// field, four per register; its E-step address is that byte plus the table's LDS base.
constexpr int kCellsPerWord = 4;
static_assert(kMaxCells * kCellBytes <= 256, "cell offsets fit a byte");
template <int E>
struct CellWords {
  static constexpr int value = (E + kCellsPerWord - 1) / kCellsPerWord;
};
typedef __attribute__((address_space(3))) unsigned char lds_byte;
__device__ __forceinline__ uint32_t lds_address(unsigned char* p) {
  return static_cast<uint32_t>(reinterpret_cast<size_t>((lds_byte*)p));
}
__device__ __forceinline__ float2 lds_read_float2(uint32_t a) {
  const unsigned long long v = *reinterpret_cast<const __attribute__((address_space(3))) unsigned long long*>(
      static_cast<size_t>(a));
  return make_float2(__uint_as_float(static_cast<uint32_t>(v)), __uint_as_float(static_cast<uint32_t>(v >> 32)));
}
// Lane-private fp64 bins, optionally shared by the lanes l, l + 64/kBinShare, ... of a
// wave.  Sharers sit in different 16-lane groups of an LDS instruction, so they never
// collide on a bank within a cycle, and the instruction's fixed lane-group order keeps
// the accumulation order (and the fp64 result) deterministic.
#ifndef ANY4_BIN_SHARE
#define ANY4_BIN_SHARE 2
#endif
constexpr int kBinShare = ANY4_BIN_SHARE;
constexpr int kBinCols = kWave / kBinShare;
constexpr size_t kBinBytesPerWave = 2 * kMaxClusters * kBinCols * sizeof(double);

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

// Wave-level reductions and scans with DPP lane moves (VALU latency, no LDS round
// trip).  Controls: quad_perm [1,0,3,2] = 0xB1, [2,3,0,1] = 0x4E, row_half_mirror
// 0x141, row_mirror 0x140, row_shr:n 0x110+n, row_bcast:15 0x142, row_bcast:31 0x143.
// Lanes without a source lane (row shifts) read 0; rows outside ROW_MASK keep 0.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xF, ROW_MASK == 0xF);
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(dpp<CTRL, ROW_MASK>(__float_as_int(v)));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ unsigned long long dpp64(unsigned long long v) {
  const uint32_t lo = static_cast<uint32_t>(dpp<CTRL, ROW_MASK>(static_cast<int>(v)));
  const uint32_t hi = static_cast<uint32_t>(dpp<CTRL, ROW_MASK>(static_cast<int>(v >> 32)));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ double dppd(double v) {
  return __longlong_as_double(
      static_cast<long long>(dpp64<CTRL, ROW_MASK>(static_cast<unsigned long long>(__double_as_longlong(v)))));
}
__device__ __forceinline__ float readlane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
__device__ __forceinline__ double readlane_d(double v, int l) {
  const long long b = __double_as_longlong(v);
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(b >> 32), l));
  return __longlong_as_double(static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo));
}
// A double holding an exact integer in [0, 2^52) as u64: adding 2^52 is exact and leaves
// the integer in the mantissa bits (two ops instead of a general conversion).
__device__ __forceinline__ unsigned long long exact_u64(double v) {
  return static_cast<unsigned long long>(__double_as_longlong(v + 4503599627370496.0)) -
         0x4330000000000000ull;
}
// Fixed-point Eq. 23 terms (rows of 2-16 waves): a term t with |t| < 2^51 becomes the
// nearest integer by one fused add of 1.5 * 2^52, whose result lies in [2^52, 2^53) where
// doubles are spaced by 1; the bit pattern of that double minus the constant's is the
// integer in two's complement (one op on the high word).  Integer sums do not depend on
// their order, so every wave of a row can add into the same bins.
constexpr double kFixBias = 6755399441055744.0;  // 1.5 * 2^52
constexpr unsigned long long kFixBiasBits = 0x4338000000000000ull;
__device__ __forceinline__ unsigned long long fix_term(double u, double v) {
  return static_cast<unsigned long long>(__double_as_longlong(__builtin_fma(u, v, kFixBias))) -
         kFixBiasBits;
}
__device__ __forceinline__ unsigned long long readlane_u64(unsigned long long v, int l) {
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), l));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v >> 32), l));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}

// max/min of the wave, uniform result
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));  // every lane of a row now holds the row's max
  return fmaxf(fmaxf(readlane_f(v, 0), readlane_f(v, 16)), fmaxf(readlane_f(v, 32), readlane_f(v, 48)));
}
__device__ __forceinline__ float wave_min(float v) {
  v = fminf(v, dppf<0xB1>(v));
  v = fminf(v, dppf<0x4E>(v));
  v = fminf(v, dppf<0x141>(v));
  v = fminf(v, dppf<0x140>(v));
  return fminf(fminf(readlane_f(v, 0), readlane_f(v, 16)), fminf(readlane_f(v, 32), readlane_f(v, 48)));
}
// fp64 sum of the wave in a fixed order, uniform result
__device__ __forceinline__ double wave_sum_f64(double v) {
  v += dppd<0xB1>(v);
  v += dppd<0x4E>(v);
  v += dppd<0x141>(v);
  v += dppd<0x140>(v);
  return (readlane_d(v, 0) + readlane_d(v, 16)) + (readlane_d(v, 32) + readlane_d(v, 48));
}
// inclusive prefix sums over the wave's lanes
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v) {
  v += dpp64<0x111>(v);
  v += dpp64<0x112>(v);
  v += dpp64<0x114>(v);
  v += dpp64<0x118>(v);
  v += dpp64<0x142, 0xA>(v);
  v += dpp64<0x143, 0xC>(v);
  return v;
}
// inclusive prefix sums over lanes 0..N-1 (N <= 32; lanes past N hold partial sums)
template <int N>
__device__ __forceinline__ double lanes_incl_scan_f64(double v) {
  static_assert(N <= 32, "two DPP rows at most");
  v += dppd<0x111>(v);
  v += dppd<0x112>(v);
  if constexpr (N > 4) v += dppd<0x114>(v);
  if constexpr (N > 8) v += dppd<0x118>(v);
  if constexpr (N > 16) v += dppd<0x142, 0xA>(v);
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

// Bisection over floats by an integer key that orders like the values: for
// non-negative floats the bit pattern itself; with SIGNED (symmetric scaling, where the
// scaled weights can be negative) the sign-flipped pattern, so that -0 sits just below
// +0 and negative values order by their magnitude reversed.
template <bool SIGNED>
__device__ __forceinline__ uint32_t order_key(float f) {
  const uint32_t b = __float_as_uint(f);
  if (!SIGNED) return b;
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
template <bool SIGNED>
__device__ __forceinline__ float key_float(uint32_t k) {
  if (!SIGNED) return __uint_as_float(k);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// Smallest fp32 x in [cl, cr] (cl < cr; both >= 0 unless SIGNED) at which R wins.  The
// rule is monotone in x on that interval (left distance non-decreasing, right
// non-increasing under monotone rounding), so the winners form a suffix of the ordered
// keys.  The answer lies within a few ulps of the rounded midpoint: the five keys
// mb-2..mb+2 are tested independently, and when mb-2 loses and mb+2 wins the answer is
// mb-2 plus the number of losers.  Otherwise a bisection over the keys decides (exact).
template <bool SIGNED>
__device__ float switch_point(float cl, int il, float cr, int ir) {
  uint32_t lo = order_key<SIGNED>(cl), hi = order_key<SIGNED>(cr);
  const float mid = cl + 0.5f * (cr - cl);
  const uint32_t mb = order_key<SIGNED>(mid);
  if (mb >= lo + 2 && mb + 2 <= hi) {
    uint32_t losers = 0;
    bool w0 = false, w4 = false;
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const bool w = right_wins(key_float<SIGNED>(mb - 2 + j), cl, il, cr, ir);
      losers += w ? 0u : 1u;
      if (j == 0) w0 = w;
      if (j == 4) w4 = w;
    }
    if (!w0 && w4) return key_float<SIGNED>(mb - 2 + losers);
  }
  if (mb >= lo + 2 && !right_wins(key_float<SIGNED>(mb - 2), cl, il, cr, ir)) lo = mb - 1;
  if (mb + 2 <= hi && right_wins(key_float<SIGNED>(mb + 2), cl, il, cr, ir)) hi = mb + 2;
  // invariant: every x below lo loses (or lo == cl), and hi wins (or hi == cr)
  for (int guard = 0; guard < 40 && lo < hi; ++guard) {
    const uint32_t m = lo + ((hi - lo) >> 1);
    if (right_wins(key_float<SIGNED>(m), cl, il, cr, ir))
      hi = m;
    else
      lo = m + 1;
  }
  return key_float<SIGNED>(hi);
}

__device__ __forceinline__ float switch_point_any(float cl, int il, float cr, int ir, bool sgn) {
  return sgn ? switch_point<true>(cl, il, cr, ir) : switch_point<false>(cl, il, cr, ir);
}

// Fixed grid over the scaled range: cell h holds x with x + off in [h/2, (h+1)/2), where
// off = 0 for asymmetric scaling (w_S in [0, 2^n - 1]) and 2^(n-1) for symmetric scaling
// (w_S in [-2^(n-1), 2^(n-1)]).  fl(x + off) * 2 is monotone in x, so the cell is too;
// values past either end clamp into the end cells.  With at most
// 32 cells of 8 bytes the whole table spans each LDS bank pair once, so the gathers of
// the E-step are free of bank conflicts (equal cells are broadcast).
__device__ __forceinline__ uint32_t cell_of(float x, int G, float off) {
  const float y = (off != 0.0f) ? x + off : x;
  const int h = static_cast<int>(y * static_cast<float>(kCellsPerUnit));
  return static_cast<uint32_t>(h < 0 ? 0 : (h < G ? h : G - 1));
}

// Wave 0 only: from S.c (k values), build the sorted distinct values, their lowest
// draw index, the switch points S.thr[0..U-2] (+inf beyond) and their cells.  The
// centroids are broadcast to uniform registers; each lane ranks its own centroid.
// Lane t < U - 1 returns switch point t and its cell in (t_out, tc_out), lane p < U the
// sorted value p and its draw index in (sv_out, si_out); returns U.
__device__ int build_structure(Smem& S, int k, int G, float off, int lane, float& t_out, uint32_t& tc_out,
                               float& sv_out, int& si_out) {
  const float inf = __builtin_huge_valf();
  float ct = (lane < k) ? S.c[lane] : inf;
  if (ct == 0.0f) ct = 0.0f;  // -0 -> +0 so that bit patterns order like values
  float cu[kMaxClusters];
#pragma unroll
  for (int u = 0; u < kMaxClusters; ++u) cu[u] = readlane_f(ct, u);
  bool first = lane < k;
#pragma unroll
  for (int u = 0; u < kMaxClusters; ++u)
    if (u < lane && cu[u] == ct) first = false;
  const unsigned long long fm = __ballot(first);
  int less = 0;
#pragma unroll
  for (int u = 0; u < kMaxClusters; ++u)
    if (((fm >> u) & 1ull) && cu[u] < ct) ++less;
  const int U = __popcll(fm);
  if (first) {
    S.sv[less] = ct;
    S.sidx[less] = lane;
  }
  wave_lds_fence();
  float t = inf;
  uint32_t tc = kMaxCells;
  if (lane + 1 < U) {
    t = switch_point_any(S.sv[lane], S.sidx[lane], S.sv[lane + 1], S.sidx[lane + 1], off != 0.0f);
    tc = cell_of(t, G, off);
  }
  sv_out = (lane < U) ? S.sv[lane] : inf;
  si_out = (lane < U) ? S.sidx[lane] : 0;
  if (lane < kMaxClusters + 4) {
    S.thr[lane] = t;
    S.tcell[lane] = tc;
  }
  if (lane == 0) S.n_unique = U;
  wave_lds_fence();
  t_out = t;
  tc_out = tc;
  return U;
}

// exclusive prefix sums of a u32 over the wave's lanes
__device__ __forceinline__ uint32_t wave_excl_scan_u32(uint32_t v) {
  uint32_t s = v;
  s += static_cast<uint32_t>(dpp<0x111>(static_cast<int>(s)));
  s += static_cast<uint32_t>(dpp<0x112>(static_cast<int>(s)));
  s += static_cast<uint32_t>(dpp<0x114>(static_cast<int>(s)));
  s += static_cast<uint32_t>(dpp<0x118>(static_cast<int>(s)));
  s += static_cast<uint32_t>(dpp<0x142, 0xA>(static_cast<int>(s)));
  s += static_cast<uint32_t>(dpp<0x143, 0xC>(static_cast<int>(s)));
  return s - v;
}

// Wave 0, right after build_structure: the per-cell table for this round.  For cell h,
// `position` counts the switch points in earlier cells (all below any x of cell h, by
// monotonicity of cell_of), and T is the switch point inside the cell (+inf if none),
// so the cluster position of x is position + [x >= T].  The switch points' cells are
// OR-ed into a 32-bit mask across the wave; lane h < 32 fills cell h with the popcount
// of the mask below it, then each switch point writes itself into its cell.  A cell
// holding two switch points (the mask then has fewer bits than switch points) makes the
// round use the binary search (S.use_table = 0).
static_assert(kMaxCells <= 32, "one mask bit per cell");
__device__ __forceinline__ void build_table(Smem& S, unsigned char* table, int lane, float t,
                                            uint32_t tc, int U) {
  const bool owner = lane + 1 < U;
  uint32_t m = owner ? (1u << tc) : 0u;  // switch points are in lanes 0..14 (one DPP row)
  m |= static_cast<uint32_t>(dpp<0x111>(static_cast<int>(m)));  // row_shr:1
  m |= static_cast<uint32_t>(dpp<0x112>(static_cast<int>(m)));  // row_shr:2
  m |= static_cast<uint32_t>(dpp<0x114>(static_cast<int>(m)));  // row_shr:4
  m |= static_cast<uint32_t>(dpp<0x118>(static_cast<int>(m)));  // row_shr:8
  const uint32_t mask = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(m), 15));
  if (lane < kMaxCells) {
    const uint32_t below = __popc(mask & ((1u << lane) - 1u));
    reinterpret_cast<float2*>(table)[lane] = make_float2(__builtin_huge_valf(), __uint_as_float(below));
  }
  wave_lds_fence();
  if (owner) reinterpret_cast<float*>(table)[tc * (kCellBytes / 4)] = t;
  if (lane == 0) S.use_table = (__popc(mask) == U - 1) ? 1 : 0;
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
// `in_flight` runs while the loads are outstanding: with OVERLAP, in the common case (a
// full lane of 16-byte aligned bf16 data) every load of W and E|x| is issued first, then
// `in_flight`, then the conversions, so no load waits for another; otherwise (and in the
// 128-VGPR instances, where the raw words would spill) it runs after the loads.
template <int E, bool OVERLAP, typename F>
__device__ __forceinline__ void load_row(const MatDesc& M, int64_t row, int K, int col0,
                                         float (&x)[E], float (&act)[E], F&& in_flight) {
  const bool full = col0 + E <= K;
  const int nv = K - col0;  // valid columns of this lane (may be <= 0 or >= E)
  const bool act_vec = full && (K & 3) == 0 && ((reinterpret_cast<uintptr_t>(M.act) & 15) == 0);
  if (OVERLAP && M.dtype == 1 && act_vec && (K & 7) == 0 &&
      ((reinterpret_cast<uintptr_t>(M.w) & 15) == 0)) {
    const uint4* wsrc = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(M.w) + row * (int64_t)K + col0);
    const float4* asrc = reinterpret_cast<const float4*>(M.act + col0);
    uint4 wr[E / 8];
    float4 ar[E / 4];
#pragma unroll
    for (int v = 0; v < E / 8; ++v) wr[v] = wsrc[v];
#pragma unroll
    for (int v = 0; v < E / 4; ++v) ar[v] = asrc[v];
    in_flight();
#pragma unroll
    for (int v = 0; v < E / 8; ++v) {
      const uint32_t w4[4] = {wr[v].x, wr[v].y, wr[v].z, wr[v].w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        x[8 * v + 2 * h] = bf16_bits_to_float(w4[h] & 0xFFFFu);
        x[8 * v + 2 * h + 1] = bf16_bits_to_float(w4[h] >> 16);
      }
    }
#pragma unroll
    for (int v = 0; v < E / 4; ++v) {
      act[4 * v] = ar[v].x;
      act[4 * v + 1] = ar[v].y;
      act[4 * v + 2] = ar[v].z;
      act[4 * v + 3] = ar[v].w;
    }
    return;
  }
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
      for (int m = 0; m < E; ++m) x[m] = (m < nv) ? bf16_bits_to_float(src[m]) : 0.0f;
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
      for (int m = 0; m < E; ++m) x[m] = (m < nv) ? src[m] : 0.0f;
    }
  }
  const float* asrc = M.act + col0;
  if (act_vec) {
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
    for (int m = 0; m < E; ++m) act[m] = (m < nv) ? asrc[m] : 0.0f;
  }
  in_flight();
}

// Scaling of a call: Qmax - Qmin = qr = 2^n - 1 (Eq. 2), Qmax = qmax = 2^(n-1) for the
// symmetric variant (Eq. 3), and the variant word (sample-weight term, symmetric bit).
struct ScaleParams {
  float qr;
  float qmax;
  int32_t variant;
};

// Eq. 1-2 (or Eq. 3) on one group held in registers [m0, m0+G), then the sample weights
// of Eq. 23 (alpha * E|x|, or the ablated terms of Appendix C.1: E|x| alone, or 1).
// Writes alpha/beta of the group (fp32 for the scale stage, fp16 otherwise).
template <int MODE, bool RECIP>
__device__ __forceinline__ void finish_group(float mn, float mx, const ScaleParams& sp, float* x,
                                             float* act, int n, bool& bad, const MatDesc& M,
                                             int64_t row, int64_t gidx, int64_t n_groups,
                                             bool writer) {
  const bool sym = (sp.variant & kVarSymmetric) != 0;
  // symmetric: max|w| of the group is the larger magnitude of its extremes
  const float alpha = sym ? fmaxf(fabsf(mn), fabsf(mx)) / sp.qmax : (mx - mn) / sp.qr;
  const float beta = sym ? 0.0f : mn;
  const int wmode = sp.variant & kVarWeightMask;
  if (!is_finite(alpha)) bad = true;
  // w_S = fl32(diff / alpha) without a division per element: alpha is one value per
  // group, so its reciprocal is taken once in fp64 and each quotient is
  // fl32(fl64(diff * fl64(1 / alpha))).  The fp64 product lies within 2^-52 (relative)
  // of the exact quotient, and a quotient of two fp32 values that is not itself an fp32
  // value lies at least 2^-49 (relative) from every fp32 rounding midpoint, so rounding
  // it to fp32 gives the correctly rounded quotient the division would.
  // RECIP is set where a lane holds one group (groups at least as wide as a lane's
  // columns); groups narrower than that keep one fp32 division per element, one in flight
  // at a time, since several reciprocals held at once would cost registers.
  const double rinv = (RECIP && alpha > 0.0f) ? 1.0 / static_cast<double>(alpha) : 0.0;
  for (int m = 0; m < n; ++m) {
    if (!RECIP) asm volatile("" : "+v"(x[m]), "+v"(act[m]));
    float ws = 0.0f;
    if (alpha > 0.0f) {
      const float diff = x[m] - beta;
      ws = RECIP ? static_cast<float>(static_cast<double>(diff) * rinv) : diff / alpha;
    }
    // x and E|x| are finite (checked on load) and so is alpha (checked above), so a is
    // never NaN, w_S is bounded and a * w_S is finite unless a is huge: the row's
    // largest a is checked against kAMax once, after the row vote
    const float a = (wmode == 0) ? alpha * act[m] : (wmode == 1 ? act[m] : 1.0f);
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
__device__ __forceinline__ void scale_narrow(float (&x)[E], float (&act)[E], const ScaleParams& sp, int K,
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
      finish_group<MODE, false>(mn, mx, sp, &x[lg * G], &act[lg * G], G, bad, M, row,
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
__device__ __forceinline__ void scale_wide(float (&x)[E], float (&act)[E], const ScaleParams& sp, int K,
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
    // lanes of a group are aligned: combine pairs, quads, 8 and 16 with DPP moves
    if (L >= 2) { mn = fminf(mn, dppf<0xB1>(mn)); mx = fmaxf(mx, dppf<0xB1>(mx)); }
    if (L >= 4) { mn = fminf(mn, dppf<0x4E>(mn)); mx = fmaxf(mx, dppf<0x4E>(mx)); }
    if (L >= 8) { mn = fminf(mn, dppf<0x141>(mn)); mx = fmaxf(mx, dppf<0x141>(mx)); }
    if (L >= 16) { mn = fminf(mn, dppf<0x140>(mn)); mx = fmaxf(mx, dppf<0x140>(mx)); }
    for (int s = 16; s < L; s <<= 1) {
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
    finish_group<MODE, true>(mn, mx, sp, x, act, E, bad, M, row, col0 / g, K / g, (col0 % g) == 0);
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) {
      x[m] = 0.0f;
      act[m] = 0.0f;
    }
  }
}

// ---------------------------------------------------------------------------------
// Lane l's x[m] for a wave-uniform m and l: a binary search over m (uniform branches)
// ending in one readlane, so no vector register holds a copy of x.
template <int LO, int N, int E>
__device__ __forceinline__ float readlane_elem(const float (&x)[E], int m, int l) {
  if constexpr (N == 1) {
    return readlane_f(x[LO], l);
  } else {
    if (m < LO + N / 2) return readlane_elem<LO, N / 2, E>(x, m, l);
    return readlane_elem<LO + N / 2, N - N / 2, E>(x, m, l);
  }
}

// The k-means++ sampling weights of a lane's E elements: in registers, or, for rows of
// 5-16 waves (1024-lane workgroups, 128 VGPRs, where they would spill), in the wave's
// bin area, which seeding does not use (element m of lane l at word m * 64 + l, so a
// wave's accesses to one m hit 64 consecutive words).  Register-held weights are copied
// to that layout with every CDF pass, where the owner of a pick reads them.
template <int E, bool IN_LDS>
struct SeedWeights {
  float r[IN_LDS ? 1 : E];
  float* l;  // this lane's weight m at l[m * kWave]
  __device__ __forceinline__ float& operator[](int m) {
    if constexpr (IN_LDS)
      return l[m * kWave];
    else
      return r[m];
  }
};

// ---------------------------------------------------------------------------------
// One pass over the lane's elements with the current centroids.  The cluster
// position comes from the cell table (TABLE) or the binary search; ACCUM adds the two
// Eq. 23 sums into lane-private fp64 bins (address pos*64 + lane: conflict-free;
// (double)a * (double)w_S is exact, so only the order of the fp64 additions differs
// from a sequential sum); STEP also stores the assignment and sums the objective;
// FINAL packs the codes and sums the objective.
enum PassKind { PASS_ACCUM = 0, PASS_STEP = 1, PASS_FINAL = 2 };

// fp64 conversion tied to the round index `tok` (an operand the instruction ignores):
// the compiler cannot move it out of the round loop, where the conversions of the whole
// resident row would stay live in 128 registers, and needs no copy of the source.
__device__ __forceinline__ double cvt_f64_in_round(float v, int tok) {
  double r;
  asm("v_cvt_f64_f32 %0, %1" : "=v"(r) : "v"(v), "s"(tok));
  return r;
}

template <int E, int KIND, bool TABLE, bool FIX>
__device__ __forceinline__ double element_pass(float (&x)[E], float (&a)[E],
                                               const uint32_t (&cw)[CellWords<E>::value], const Smem& S,
                                               const unsigned char* table, double* bins, int lane,
                                               uint8_t* assign_row, uint32_t (&packed)[E / 8],
                                               int n_valid, int tok) {
#ifndef ANY4_CHUNK
#define ANY4_CHUNK 8
#endif
  constexpr int CH = ANY4_CHUNK;  // elements whose table reads are in flight together
  const float t7 = uniform_f(S.thr[7]);
  const uint32_t tbase = lds_address(const_cast<unsigned char*>(table));
  double J = 0.0;
#pragma unroll
  for (int m0 = 0; m0 < E; m0 += CH) {
    // the chunk's packed cell words, re-declared opaque so that they stay packed (their
    // table addresses are not hoisted out of the round loop into 32 registers)
    constexpr int NWC = (CH + kCellsPerWord - 1) / kCellsPerWord + 1;
    const int W0 = m0 / kCellsPerWord, W1 = (m0 + CH - 1) / kCellsPerWord;
    uint32_t cwc[NWC];
#pragma unroll
    for (int i = 0; i < NWC; ++i) {
      if (W0 + i <= W1) {
        cwc[i] = cw[W0 + i];
        asm volatile("" : "+v"(cwc[i]));
      }
    }
    int pos[CH];
    if (TABLE) {
      float2 e[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int m = m0 + i;
        const uint32_t w = cwc[m / kCellsPerWord - W0];
        e[i] = lds_read_float2(tbase + ((w >> (8 * (m % kCellsPerWord))) & 0xFFu));
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const float xm = x[m0 + i];
        pos[i] = static_cast<int>(__float_as_uint(e[i].y)) + (xm >= e[i].x ? 1 : 0);
      }
    } else {
#pragma unroll
      for (int i = 0; i < CH; ++i) pos[i] = sorted_position(x[m0 + i], t7, S.thr);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int m = m0 + i;
      const double ad = cvt_f64_in_round(a[m], tok);
      const double xd = cvt_f64_in_round(x[m], tok);
      if (KIND != PASS_FINAL) {
        double* b = bins + pos[i] * kBinCols + (lane & (kBinCols - 1));
        if (FIX) {
          // a is held as a * 2^sigma (< 2^43): S0 takes round(4 a), S1 round(a w_S), both
          // far below the 2^51 of fix_term (4 is an inline operand of the fused add)
          unsigned long long* bu = reinterpret_cast<unsigned long long*>(b);
          atomicAdd(bu, fix_term(ad, 4.0));
          atomicAdd(bu + kMaxClusters * kBinCols, fix_term(ad, xd));
        } else {
          atomicAdd(b, ad);
          atomicAdd(b + kMaxClusters * kBinCols, ad * xd);
        }
      }
      if (KIND != PASS_ACCUM) {
        const int q = S.sidx[pos[i]];
        const double d = xd - static_cast<double>(S.sv[pos[i]]);
        J += ad * d * d;
        if (KIND == PASS_STEP && m < n_valid) assign_row[m] = static_cast<uint8_t>(q);
        if (KIND == PASS_FINAL) packed[m / 8] |= static_cast<uint32_t>(q) << (4 * (m % 8));
      }
    }
  }
  return J;
}

// Reduce this wave's bins into 32 slot totals (S0[0..15], S1[0..15]).  The bins are
// never cleared: they accumulate over the rounds, and a round's sums are this total
// minus the previous round's (an untouched slot reads back bit-identical, so it gives
// exactly 0).  Lane l sums half of slot l>>1's columns in a fixed rotated order that puts
// the 16-byte reads of any 8 or 16 consecutive lanes on distinct banks.
__device__ __forceinline__ double reduce_bins(const double* bins, int lane) {
  asm volatile("" : "+v"(lane));  // recompute the addresses per round instead of holding them
  constexpr int CH = kBinCols / 4;  // double2 chunks per half slot
  const int slot = lane >> 1, half = lane & 1;
  const double2* src =
      reinterpret_cast<const double2*>(bins + slot * kBinCols + half * (kBinCols / 2));
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int j = (i + (lane >> 1) + (CH / 2) * half) & (CH - 1);
    const double2 v = src[j];
    s += v.x;
    s += v.y;
  }
  const double other = dppd<0xB1>(s);
  return half ? other + s : s + other;  // same order in both lanes of the pair
}

// The same reduction over fixed-point bins (mod 2^64; the round's sums are exact).
__device__ __forceinline__ unsigned long long reduce_bins_fix(const double* bins, int lane) {
  asm volatile("" : "+v"(lane));
  constexpr int CH = kBinCols / 4;
  const int slot = lane >> 1, half = lane & 1;
  const ulonglong2* src = reinterpret_cast<const ulonglong2*>(bins + slot * kBinCols + half * (kBinCols / 2));
  unsigned long long s = 0;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int j = (i + (lane >> 1) + (CH / 2) * half) & (CH - 1);
    const ulonglong2 v = src[j];
    s += v.x;
    s += v.y;
  }
  return s + dpp64<0xB1>(s);
}

__device__ __forceinline__ void zero_bins(double* bins, int lane) {
  asm volatile("" : "+v"(lane));
  constexpr int PER_LANE = 2 * kMaxClusters * kBinCols / kWave;  // doubles per lane
  double2* dst = reinterpret_cast<double2*>(bins + lane * PER_LANE);
#pragma unroll
  for (int i = 0; i < PER_LANE / 2; ++i) dst[i] = make_double2(0.0, 0.0);
}

// Wave 0, after every wave has published its reduced bins in S.wred: the Eq. 23 update
// and the next round's structure.  Lane p < U holds sorted value p (sv) and its draw
// index (si) from the previous structure; it sums S0 and S1 of position p over the waves
// in wave order, divides in fp64 and rounds to fp32 (an empty cluster keeps its value).
// When every draw index is its own position (U == k) and the new values are still
// strictly increasing by position, the sorted order and the lowest-index map are
// unchanged: only the values and the switch points are recomputed, the right neighbour
// coming from the next lane by DPP.  Otherwise the structure is rebuilt from the
// draw-order centroids.  Returns U; (t, tc) as in build_structure.  `same` tells whether
// every centroid kept its bits: then the next round's assignment, and so its sums, are
// this round's, and every later round would give the same centroids again.
__device__ __forceinline__ int update_and_structure(Smem& S, int nw, int k, int G, float off, int lane, int U,
                                                    float& sv, int& si, float& t,
                                                    uint32_t& tc, bool& same) {
  float cn = sv;
  double s0 = 0.0, s1 = 0.0;
  if (nw <= 4) {
    if (lane < U) {
      s0 = S.wred[0][lane];
      s1 = S.wred[0][kMaxClusters + lane];
      for (int w = 1; w < nw; ++w) {
        s0 += S.wred[w][lane];
        s1 += S.wred[w][kMaxClusters + lane];
      }
    }
  } else {
    // many waves: lanes p + 16 j (j < 4) add waves j, j + 4, j + 8, ... of position p, then
    // lane p adds the four partials in j order (a fixed order, shorter than nw dependent
    // reads); positions p >= U add what their bins hold (zeros) and are not used
    const int p = lane & (kMaxClusters - 1), j = lane >> 4;
    for (int w = j; w < nw; w += 4) {
      s0 += S.wred[w][p];
      s1 += S.wred[w][kMaxClusters + p];
    }
    const double a0 = __shfl(s0, p + 16), a1 = __shfl(s1, p + 16);
    const double b0 = __shfl(s0, p + 32), b1 = __shfl(s1, p + 32);
    const double c0 = __shfl(s0, p + 48), c1 = __shfl(s1, p + 48);
    s0 = ((s0 + a0) + b0) + c0;
    s1 = ((s1 + a1) + b1) + c1;
  }
  if (lane < U) {
    if (s0 > 0.0) cn = static_cast<float>(s1 / s0);
    S.c[si] = cn;
  }
  same = __ballot(lane < U && __float_as_uint(cn) != __float_as_uint(sv)) == 0ull;
  const float cnext = dppf<0x101>(cn);  // row_shl:1, value of lane + 1 (lanes < 16)
  const bool out_of_order = lane + 1 < U && !(cn < cnext);
  if (U == k && __ballot(out_of_order) == 0ull) {
    const int inext = dpp<0x101>(si);
    t = __builtin_huge_valf();
    tc = kMaxCells;
    if (lane + 1 < U) {
      t = switch_point_any(cn, si, cnext, inext, off != 0.0f);
      tc = cell_of(t, G, off);
    }
    sv = cn;
    if (lane < U) S.sv[lane] = cn;
    if (lane < kMaxClusters + 4) {
      S.thr[lane] = t;
      S.tcell[lane] = tc;
    }
    wave_lds_fence();
    return U;
  }
  wave_lds_fence();
  return build_structure(S, k, G, off, lane, t, tc, sv, si);
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
// Occupancy target per element count: 32 elements per lane fit 3 waves per SIMD.
template <int E>
struct WavesPerEU {
  static constexpr int value = (E == 32) ? 3 : 0;
};

// WIDE: the group is at least as wide as a lane's E columns (one group per lane); the
// kernel is instantiated separately for narrower groups so that neither carries the
// other's scaling code.  VAR: the instance that honours the method-variant word and the
// restart index; without it every variant branch folds away and the default path keeps
// its own register allocation.
// The variant instance for narrow groups is held to 2 waves per SIMD instead of 3: at
// 168 VGPRs it spilled ~3700 registers around the narrow-group scaling cases; at 2 waves
// it spills none and runs 17-35% faster (group 8 and 16 variants on 14336 x 4096).
// The 1024-lane instance (NWMAX 16: rows of 5 to 16 waves, and default-path rows of 2 to 4
// waves) is capped at 128 VGPRs: such a workgroup may put 4 waves on every SIMD.
template <int E, int NWMAX, int MODE, bool WIDE, bool VAR>
__global__ __launch_bounds__(kWave* NWMAX)
__attribute__((amdgpu_waves_per_eu(NWMAX > 8 ? 4
                                   : (VAR && !WIDE && WavesPerEU<E>::value > 2)
                                       ? 2
                                       : (WavesPerEU<E>::value == 0 ? 1 : WavesPerEU<E>::value))))
void any4_rows_kernel(const LaunchArgs args) {
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
  const int32_t variant = VAR ? args.variant : 0;
  const int restart = VAR ? args.restart : 0;
  const ScaleParams sp{qr, static_cast<float>(k / 2), variant};
  const int init = (variant >> kVarInitShift) & 3;
  // symmetric scaling puts w_S in [-k/2, k/2]: the cell grid starts at -k/2
  const float cell_off = (variant & kVarSymmetric) ? static_cast<float>(k / 2) : 0.0f;
  const int col0 = tid * E;

  const int n_valid = (K - col0 < E) ? (K - col0 > 0 ? K - col0 : 0) : E;  // valid columns here
  float xv[E], av[E];
  // the k-means++ draws, one Philox4x32-10 block per (row, step), computed while the row
  // loads (restart r uses the counters t + 16 r); read after the row vote's barrier
  load_row<E, (NWMAX <= 8)>(M, row, K, col0, xv, av, [&]() {
    if ((MODE == MODE_FULL || MODE == MODE_SEED) && init != INIT_UNIFORM && tid < k) {
      const uint64_t rid = static_cast<uint64_t>(M.row_offset + row);
      uint32_t c[4] = {static_cast<uint32_t>(rid), static_cast<uint32_t>(tid + 16 * restart),
                       static_cast<uint32_t>(M.matrix_index), static_cast<uint32_t>(rid >> 32)};
      philox4x32_10(c, static_cast<uint32_t>(args.seed), static_cast<uint32_t>(args.seed >> 32));
      S.u[tid] = (static_cast<unsigned long long>(c[1]) << 32) | c[0];
    }
  });

  bool bad = false;
  if (n_valid == E) {
#pragma unroll
    for (int m = 0; m < E; ++m)
      if (!is_finite(xv[m]) || !(av[m] >= 0.0f && av[m] <= __FLT_MAX__)) bad = true;
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m)
      if (m < n_valid && (!is_finite(xv[m]) || !(av[m] >= 0.0f && av[m] <= __FLT_MAX__))) bad = true;
  }

  // ---- Eq. 1-2 scaling and Eq. 23 sample weights
  if constexpr (WIDE) {
    scale_wide<E, MODE>(xv, av, sp, K, col0, bad, M, row, g, S, lane, wave, nw);
  } else {
    switch (g) {
      case 2: scale_narrow<E, 2, MODE>(xv, av, sp, K, col0, bad, M, row, g); break;
      case 4: scale_narrow<E, 4, MODE>(xv, av, sp, K, col0, bad, M, row, g); break;
      case 8: if constexpr (E > 8) scale_narrow<E, 8, MODE>(xv, av, sp, K, col0, bad, M, row, g); break;
      case 16: if constexpr (E > 16) scale_narrow<E, 16, MODE>(xv, av, sp, K, col0, bad, M, row, g); break;
      case 32: if constexpr (E > 32) scale_narrow<E, 32, MODE>(xv, av, sp, K, col0, bad, M, row, g); break;
      default: break;
    }
  }

  if (MODE == MODE_SCALE) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
      if (m < n_valid) {
        M.ws_out[row * K + col0 + m] = xv[m];
        M.a_out[row * K + col0 + m] = av[m];
      }
    }
    return;
  }

  // a row is rejected when any lane found a bad value (per-wave votes in LDS; the
  // runtime's block vote would add static shared memory in front of the dynamic one).
  // The same exchange carries the row's largest sample weight and the range of its
  // scaled weights, which set the k-means++ sampling scales.
  if (tid == 0) S.x0 = xv[0];
  float l_amax = 0.0f, l_xmin = __builtin_huge_valf(), l_xmax = -__builtin_huge_valf();
  if (n_valid == E) {
#pragma unroll
    for (int m = 0; m < E; ++m) {
      l_amax = fmaxf(l_amax, av[m]);
      l_xmin = fminf(l_xmin, xv[m]);
      l_xmax = fmaxf(l_xmax, xv[m]);
    }
  } else {
#pragma unroll
    for (int m = 0; m < E; ++m) {
      if (m < n_valid) {
        l_amax = fmaxf(l_amax, av[m]);
        l_xmin = fminf(l_xmin, xv[m]);
        l_xmax = fmaxf(l_xmax, xv[m]);
      }
    }
  }
  l_amax = wave_max(l_amax);
  l_xmin = wave_min(l_xmin);
  l_xmax = wave_max(l_xmax);
  const bool wave_bad = __ballot(bad) != 0ull;
  if (lane == 0) {
    S.bad[wave] = wave_bad ? 1 : 0;
    S.rstat[0][wave] = l_amax;
    S.rstat[1][wave] = l_xmin;
    S.rstat[2][wave] = l_xmax;
  }
  __syncthreads();
  bool row_bad = false;
  float a_max = 0.0f;
  // the first four waves' slots read at once (slots past nw are stale and dropped)
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const int bw = S.bad[w];
    const float aw = S.rstat[0][w];
    row_bad = row_bad || (w < nw && bw != 0);
    a_max = fmaxf(a_max, w < nw ? aw : 0.0f);
  }
  for (int w = 4; w < nw; ++w) {
    row_bad = row_bad || S.bad[w] != 0;
    a_max = fmaxf(a_max, S.rstat[0][w]);
  }
  a_max = uniform_f(a_max);
  row_bad = row_bad || !(a_max <= kAMax);  // a sample weight above 2^64 (or an overflow to inf)
  if (row_bad) {
    if (MODE == MODE_FULL) {
      for (int m = 0; m < E; m += 2)
        if (m < n_valid) M.codes[row * (K / 2) + (col0 + m) / 2] = 0;
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
  } else if (init == INIT_UNIFORM) {
    // Appendix C.2's uniform initialization: the integer levels, 0..2^n - 1 for
    // asymmetric scaling and 1 - 2^(n-1)..2^(n-1) (int4's -7..8) for symmetric; no draws
    if (tid < k) {
      S.c[tid] = (cell_off != 0.0f ? 1.0f - cell_off : 0.0f) + static_cast<float>(tid);
      S.picks[tid] = -1;
    }
    __syncthreads();
    if (MODE == MODE_SEED) {
      if (tid < k) {
        M.c_out[row * k + tid] = S.c[tid];
        M.picks_out[row * k + tid] = -1;
      }
      return;
    }
    if (M.picks_out && tid < k) M.picks_out[row * k + tid] = -1;
  } else {
    if (init == INIT_GREEDY && tid < k * (greedy_trials(k) - 1)) {
      // greedy candidates s >= 1 of draw t: counter word t + 16 restart + 65536 s
      const int s = 1 + tid / k, t = tid - (s - 1) * k;
      const uint64_t rid = static_cast<uint64_t>(M.row_offset + row);
      uint32_t c[4] = {static_cast<uint32_t>(rid),
                       static_cast<uint32_t>(t + 16 * restart) + 65536u * static_cast<uint32_t>(s),
                       static_cast<uint32_t>(M.matrix_index), static_cast<uint32_t>(rid >> 32)};
      philox4x32_10(c, static_cast<uint32_t>(args.seed), static_cast<uint32_t>(args.seed >> 32));
      S.gk.u[s - 1][t] = (static_cast<unsigned long long>(c[1]) << 32) | c[0];
    }
    // The sampling weights of every draw are in the wave's bin area (which seeding does
    // not use) when the owner of a pick looks for its element: rows of 5-16 waves keep
    // them there, the others keep them in registers and copy them there with each CDF pass.
    constexpr bool kPvLds = NWMAX > 8;
    static_assert(E * kWave * sizeof(float) <= kBinBytesPerWave, "weights fit the bins");
    float* const pv_area = reinterpret_cast<float*>(smem_raw + kSmemHdr + kTableBytes + wave * kBinBytesPerWave);
    SeedWeights<E, kPvLds> pv;
    pv.l = pv_area + lane;
    // Integer CDF terms floor(p * 2^ksc), ksc = 40 - floor(log2 B), for a bound B of the
    // draw's weights: the largest sample weight for the first draw, and one bound for all
    // later draws, fixed after the first pick (below).  B = 0 leaves every term 0 and the
    // centre is copied.  The weights are held scaled, pv = p * 2^ksc, so a term is
    // floor(pv): the scale is exact (pv < 2^41; a value that underflows is below 1 and
    // floors to 0 either way), and so is the floor.  From the second k-means++ draw on,
    // with ksc >= 0, the sample weights themselves carry the scale (a' = a * 2^ksc, exact,
    // undone after seeding) and pv = fl(a' * D); with ksc < 0, pv = fl(fl(a * D) * 2^ksc).
    int ksc = 0;
    bool live = a_max > 0.0f;
    if (live) {
      int e2;
      frexpf(a_max, &e2);
      ksc = 40 - (e2 - 1);
    }
#pragma unroll
    for (int m = 0; m < E; ++m) pv[m] = ldexpf(av[m], ksc);
    bool pre = false;  // av holds a * 2^ksc
    __syncthreads();
    const unsigned long long u_lane = S.u[lane & (kMaxClusters - 1)];  // draw t's Philox output in lane t
    float ct = 0.0f, c_first = 0.0f;  // the previous centre and centre 0 (uniform)
    int pick = -1;
    for (int t = 0; t < k; ++t) {
      __builtin_amdgcn_s_setprio(0);
      if (t == 1 && init != INIT_RANDOM) {
        // no later weight a_j * D_j exceeds max_j a_j * m^2, m the larger distance from
        // centre 0 to the row's extremes (D only decreases; rounding is monotone)
        float x_min = S.rstat[1][0], x_max = S.rstat[2][0];
#pragma unroll
        for (int w = 1; w < 4; ++w) {
          const float lo = S.rstat[1][w], hi = S.rstat[2][w];
          x_min = fminf(x_min, w < nw ? lo : x_min);
          x_max = fmaxf(x_max, w < nw ? hi : x_max);
        }
        for (int w = 4; w < nw; ++w) {
          x_min = fminf(x_min, S.rstat[1][w]);
          x_max = fmaxf(x_max, S.rstat[2][w]);
        }
        const float up = uniform_f(x_max) - c_first, down = c_first - uniform_f(x_min);
        const float mm = up > down ? up : down;
        const float bound = a_max * (mm * mm);
        live = bound > 0.0f;
        if (live) {
          int e2;
          frexpf(bound, &e2);
          ksc = 40 - (e2 - 1);
        }
        pre = __builtin_amdgcn_readfirstlane((live && ksc >= 0) ? 1 : 0) != 0;
        const int ka = pre ? ksc : 0;
#pragma unroll
        for (int m = 0; m < E; ++m) av[m] = ldexpf(av[m], ka);
      }
      // This draw's scaled sampling weights, then their CDF terms.  For t >= 1 the weights
      // are a_j * min_t fl((w_S_j - c_t)^2), updated from the previous centre (the min of
      // the products is the product of the min: rounding is monotone).
      // They are never NaN and never below zero (a zero may be -0), so the float order is
      // the order of their bit patterns as signed integers: the min runs as an integer op,
      // which needs no NaN quieting of its operands.  Each term floor(pv) is widened to
      // fp64 exactly (a lane's sum stays below 2^46).
      if (t > 0 && init == INIT_RANDOM) {
        // random initialization (Appendix C.2): the drawn element leaves the pool, the
        // others keep their weight a_j
        const int pm = pick - tid * E;  // no draw (pick < 0) never matches
#pragma unroll
        for (int m = 0; m < E; ++m)
          if (m == pm) pv[m] = 0.0f;
      } else if (t == 1) {
        if (pre) {
#pragma unroll
          for (int m = 0; m < E; ++m) {
            float d = xv[m] - ct;
            d = d * d;
            pv[m] = av[m] * d;
          }
        } else {
#pragma unroll
          for (int m = 0; m < E; ++m) {
            float d = xv[m] - ct;
            d = d * d;
            pv[m] = ldexpf(av[m] * d, ksc);
          }
        }
      } else if (t > 1 && !kPvLds) {
        if (pre) {
#pragma unroll
          for (int m = 0; m < E; ++m) {
            float d = xv[m] - ct;
            d = d * d;
            const int pd = __float_as_int(av[m] * d);
            pv[m] = __int_as_float(min(__float_as_int(pv[m]), pd));
          }
        } else {
#pragma unroll
          for (int m = 0; m < E; ++m) {
            float d = xv[m] - ct;
            d = d * d;
            const int pd = __float_as_int(ldexpf(av[m] * d, ksc));
            pv[m] = __int_as_float(min(__float_as_int(pv[m]), pd));
          }
        }
      }
      double lsum = 0.0;
      if (t > 1 && kPvLds && init != INIT_RANDOM) {
        // weights in LDS: the update and the CDF term in one pass, one read and one
        // write of each weight (in registers the two passes stay apart, which keeps the
        // register pressure of the fused pass off the seeding loop)
        if (pre) {
#pragma unroll
          for (int m = 0; m < E; ++m) {
            float d = xv[m] - ct;
            d = d * d;
            const int pd = __float_as_int(av[m] * d);
            const float p = __int_as_float(min(__float_as_int(pv[m]), pd));
            pv[m] = p;
            lsum += static_cast<double>(floorf(p));
          }
        } else {
#pragma unroll
          for (int m = 0; m < E; ++m) {
            float d = xv[m] - ct;
            d = d * d;
            const int pd = __float_as_int(ldexpf(av[m] * d, ksc));
            const float p = __int_as_float(min(__float_as_int(pv[m]), pd));
            pv[m] = p;
            lsum += static_cast<double>(floorf(p));
          }
        }
      } else {
#pragma unroll
        for (int m = 0; m < E; ++m) {
          lsum += static_cast<double>(floorf(pv[m]));
          if constexpr (!kPvLds) pv.l[m * kWave] = pv[m];
        }
      }
      if (!live) lsum = 0.0;
      // From here to the next draw's update the row runs a serial chain (exchange, pick
      // search, broadcast) while the other rows on the SIMD run their element passes: a
      // raised wave priority lets the chain issue first.
      __builtin_amdgcn_s_setprio(2);
        const unsigned long long ls = exact_u64(lsum);  // below 2^46
        const unsigned long long incl = wave_incl_scan_u64(ls);
        unsigned long long woff = 0, Q = readlane_u64(incl, kWave - 1);
        if (nw > 1) {
          if (lane == kWave - 1) S.ured[t & 1][wave] = incl;
          __syncthreads();
          if (nw <= 4) {
            // the four slots read at once (slots past nw hold stale values and are dropped)
            const ulonglong2 v01 = reinterpret_cast<const ulonglong2*>(S.ured[t & 1])[0];
            const ulonglong2 v23 = reinterpret_cast<const ulonglong2*>(S.ured[t & 1])[1];
            const unsigned long long v4[4] = {v01.x, v01.y, v23.x, v23.y};
            Q = 0;
#pragma unroll
            for (int w = 0; w < 4; ++w) {
              const unsigned long long v = w < nw ? v4[w] : 0ull;
              if (w < wave) woff += v;
              Q += v;
            }
          } else {
            // many waves: lane w reads wave w's total and one scan gives every prefix
            // (exact integers, so the order does not matter), instead of nw dependent reads
            const unsigned long long v = lane < nw ? S.ured[t & 1][lane] : 0ull;
            const unsigned long long inc = wave_incl_scan_u64(v);
            Q = readlane_u64(inc, nw - 1);
            woff = wave == 0 ? 0ull : readlane_u64(inc, wave - 1);
          }
        }
        const unsigned long long excl = woff + incl - ls;
      if (Q == 0) {
        // every weight is 0, or below the scale's resolution: copy (w_S[0] for the first
        // centre, centre 0 after that)
        ct = (t == 0) ? uniform_f(S.x0) : c_first;
        pick = -1;
      } else {
        // greedy k-means++ searches several candidates (s >= 1 land in S.gk); the plain
        // draw is candidate 0
        const int n_cand = (init == INIT_GREEDY && t > 0) ? greedy_trials(k) : 1;
        for (int s = 0; s < n_cand; ++s) {
          const unsigned long long r = __umul64hi(s == 0 ? readlane_u64(u_lane, t) : S.gk.u[s - 1][t], Q);
          const bool own = ls > 0 && excl <= r && r - excl < ls;
          // The owner's wave finds the element: lane m < E reads the owner lane's weight m
          // from the bin area and the first prefix past r - excl (the draw's offset inside
          // the owner's interval) marks it; the owner lane publishes its value.
          const unsigned long long bal = __ballot(own);
          if (bal != 0ull) {
            const int ol = __ffsll(static_cast<long long>(bal)) - 1;
            const unsigned long long rr = readlane_u64(r - excl, ol);
            wave_lds_fence();  // a one-wave row reads its own copies without a barrier
            const double q = (lane < E) ? static_cast<double>(floorf(pv_area[lane * kWave + ol])) : 0.0;
            const double qi = lanes_incl_scan_f64<E>(q);
            const bool hit = lane < E && qi > static_cast<double>(rr);  // exact integers below 2^47
            int ms = __ffsll(static_cast<long long>(__ballot(hit))) - 1;
            if (ms < 0) ms = E - 1;  // unreachable: the owner's prefix always crosses r
            ms = __builtin_amdgcn_readfirstlane(ms);
            const float xm = readlane_elem<0, E, E>(xv, ms, ol);
            if (lane == 0) {
              const int j = (wave * kWave + ol) * E + ms;
              if (s == 0) {
                S.pick_c = xm;
                S.pick_j = j;
              } else {
                S.gk.cand_c[s] = xm;
                S.gk.cand_j[s] = j;
              }
            }
          }
          __syncthreads();
        }
        ct = uniform_f(S.pick_c);
        pick = __builtin_amdgcn_readfirstlane(S.pick_j);
        if (n_cand > 1) {
          // each candidate's potential sum_j floor(min(p_j, a_j (w_S_j - c)^2) * 2^ksc) (the
          // weights scaled as above): exact integers (per lane below 2^47 in fp64, per row in
          // u64), compared exactly
          const int kpost = pre ? 0 : ksc;  // the scale still to apply to a product
          for (int s = 0; s < n_cand; ++s) {
            const float cs = s == 0 ? ct : S.gk.cand_c[s];
            double lp = 0.0;
#pragma unroll
            for (int m = 0; m < E; ++m) {
              float d = xv[m] - cs;
              d = d * d;
              const float pc = ldexpf(av[m] * d, kpost);
              const int pm = min(__float_as_int(pv[m]), __float_as_int(pc));
              lp += static_cast<double>(floorf(__int_as_float(pm)));
            }
            const unsigned long long tot =
                readlane_u64(wave_incl_scan_u64(exact_u64(lp)), kWave - 1);
            if (lane == 0) S.gk.pot[wave][s] = tot;
          }
          __syncthreads();
          unsigned long long best = 0;
          for (int s = 0; s < n_cand; ++s) {
            unsigned long long pot = 0;
            for (int w = 0; w < nw; ++w) pot += S.gk.pot[w][s];
            if (s == 0 || pot < best) {
              best = pot;
              if (s > 0) {
                ct = S.gk.cand_c[s];
                pick = S.gk.cand_j[s];
              }
            }
          }
          __syncthreads();  // S.gk.pot is read before the next draw writes it
        }
      }
      if (tid == 0) {
        S.c[t] = ct;
        S.picks[t] = pick;
      }
      if (t == 0) c_first = ct;
    }
    __builtin_amdgcn_s_setprio(0);
    {
      // back to the sample weights of Eq. 23 (exact: the scale only raised the exponents)
      const int ka = pre ? -ksc : 0;
#pragma unroll
      for (int m = 0; m < E; ++m) av[m] = ldexpf(av[m], ka);
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
  const int G = kCellsPerUnit * k;
  unsigned char* table = smem_raw + kSmemHdr;
  uint32_t cw[CellWords<E>::value];  // byte offset of each element's table cell, four per register
#pragma unroll
  for (int i = 0; i < CellWords<E>::value; ++i) cw[i] = 0;
#pragma unroll
  for (int m = 0; m < E; ++m)
    cw[m / kCellsPerWord] |= (cell_of(xv[m], G, cell_off) * kCellBytes) << (8 * (m % kCellsPerWord));
  // Rows of 2-16 waves sum the Eq. 23 terms in 64-bit fixed point, all waves into one
  // set of bins (wave 0's area), which wave 0 alone reduces after the round's first
  // barrier: one 8 KB reduction per round instead of one per wave.  One-wave rows keep
  // fp64 bins, reduced before that barrier.
  constexpr bool FIX = NWMAX > 1;
  double* bins = reinterpret_cast<double*>(smem_raw + kSmemHdr + kTableBytes) +
                 (FIX ? 0 : wave) * (2 * kMaxClusters * kBinCols);
  // Fixed-point scale: a * 2^sigma < 2^43 for every sample weight of the row (exact, a
  // power of two), so S0's terms round(4 a 2^sigma) stay below 2^45 and S1's
  // round(a 2^sigma w_S) below 2^47 (|w_S| < 16); a round's sums over at most 2^15
  // columns stay below 2^62 in magnitude, so the bins may wrap mod 2^64 over the rounds
  // and a round's sums are still exact.  Objectives from the scaled weights are scaled
  // back by 2^-sigma (exact).
  int sigma = 0;
  if (FIX) {
    int e_amax = 0;
    if (a_max > 0.0f) frexpf(a_max, &e_amax);
    sigma = 43 - e_amax;
#pragma unroll
    for (int m = 0; m < E; ++m) av[m] = ldexpf(av[m], sigma);
  }
  const double j_unscale = FIX ? ldexp(1.0, -sigma) : 1.0;
  uint32_t packed[E / 8];
#pragma unroll
  for (int v = 0; v < E / 8; ++v) packed[v] = 0;
  if (!FIX || wave == 0) zero_bins(bins, lane);
  double prev_total = 0.0;  // this lane's slot total after the previous round
  unsigned long long prev_fix = 0;  // the same for fixed-point bins (wave 0)
  const int rounds = (MODE == MODE_STEP) ? 1 : args.iters;
  // Per round: every wave runs its elements and publishes its reduced bins (one
  // barrier); wave 0 alone updates the centroids and prepares the next round's sorted
  // values, switch points and cell table (second barrier).
  float sv = 0.0f;  // wave 0: sorted value of position `lane`, its draw index, and U
  int si = 0, U = 0;
  if (wave == 0) {
    float t;
    uint32_t tc;
    U = build_structure(S, k, G, cell_off, lane, t, tc, sv, si);
    build_table(S, table, lane, t, tc, U);
  }
  __syncthreads();
  for (int it = 0; it < rounds; ++it) {
    const bool use_table = S.use_table != 0;
    if (MODE == MODE_STEP) {
      // E-step with its assignment and objective at c_in, then the same bin sums
      uint8_t* arow = M.assign_out + row * K + col0;
      double J = 0.0;
      if (col0 < K) {
        J = use_table ? element_pass<E, PASS_STEP, true, FIX>(xv, av, cw, S, table, bins, lane, arow,
                                                               packed, n_valid, it)
                      : element_pass<E, PASS_STEP, false, FIX>(xv, av, cw, S, table, bins, lane, arow,
                                                                packed, n_valid, it);
      }
      J = block_sum_f64(J * j_unscale, S, lane, wave, nw);
      if (tid == 0 && M.objective) M.objective[row] = J;
    } else if (col0 < K) {
      if (use_table)
        element_pass<E, PASS_ACCUM, true, FIX>(xv, av, cw, S, table, bins, lane, nullptr, packed, n_valid, it);
      else
        element_pass<E, PASS_ACCUM, false, FIX>(xv, av, cw, S, table, bins, lane, nullptr, packed, n_valid, it);
    }
    // the bin reduction and wave 0's centroid update are the round's serial chain: raised
    // priority, as in seeding, until the round's second barrier
    __builtin_amdgcn_s_setprio(2);
    if (!FIX) {
      // the reduction reads bins that other lanes of this wave just added to
      wave_lds_fence();
      const double total = reduce_bins(bins, lane);
      if ((lane & 1) == 0) S.wred[wave][lane >> 1] = total - prev_total;
      prev_total = total;
    }
    __syncthreads();
    if (wave == 0) {
      if (FIX) {
        // every wave's terms are in: the round's exact sums, in units of 2^-sigma (S0
        // scaled back from its factor 4, exactly), so that S1 / S0 is the weighted mean
        const unsigned long long total = reduce_bins_fix(bins, lane);
        if ((lane & 1) == 0) {
          const double d = static_cast<double>(static_cast<long long>(total - prev_fix));
          S.wred[0][lane >> 1] = (lane >> 1) < kMaxClusters ? d * 0.25 : d;
        }
        prev_fix = total;
        wave_lds_fence();
      }
      float t;
      uint32_t tc;
      bool same;
      U = update_and_structure(S, FIX ? 1 : nw, k, G, cell_off, lane, U, sv, si, t, tc, same);
      build_table(S, table, lane, t, tc, U);
      if (lane == 0) S.done = same ? 1 : 0;
    }
    __syncthreads();
    __builtin_amdgcn_s_setprio(0);
    // a fixed point: the remaining rounds would reproduce these centroids bit for bit
    if (S.done != 0 && !args.all_rounds) break;
  }
  if (MODE == MODE_STEP) {
    if (tid < k) M.c_out[row * k + tid] = S.c[tid];
    return;
  }

  // ---- final E-step, objective and emission (structure and table of c^iters are ready)
  const bool use_table = S.use_table != 0;
  double J = 0.0;
  if (col0 < K) {
    J = use_table ? element_pass<E, PASS_FINAL, true, FIX>(xv, av, cw, S, table, bins, lane, nullptr,
                                                            packed, n_valid, rounds)
                  : element_pass<E, PASS_FINAL, false, FIX>(xv, av, cw, S, table, bins, lane, nullptr,
                                                             packed, n_valid, rounds);
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
        if (m < n_valid) dst[m / 2] = static_cast<uint8_t>(packed[m / 8] >> (4 * (m % 8)));
    }
  }
  J = block_sum_f64(J * j_unscale, S, lane, wave, nw);
  if (tid == 0 && M.objective) M.objective[row] = J;
  if (tid < k) {
    M.lut[row * k + tid] = f16_bits(S.c[tid]);
    if (M.c_out) M.c_out[row * k + tid] = S.c[tid];
  }
}

template <int E, int NWMAX, int MODE>
void launch_kernel(const LaunchArgs& args, dim3 grid, dim3 block, size_t smem, hipStream_t stream,
                   bool wide, bool var) {
  if (wide && var)
    hipLaunchKernelGGL((any4_rows_kernel<E, NWMAX, MODE, true, true>), grid, block, smem, stream, args);
  else if (wide)
    hipLaunchKernelGGL((any4_rows_kernel<E, NWMAX, MODE, true, false>), grid, block, smem, stream, args);
  else if (var)
    hipLaunchKernelGGL((any4_rows_kernel<E, NWMAX, MODE, false, true>), grid, block, smem, stream, args);
  else
    hipLaunchKernelGGL((any4_rows_kernel<E, NWMAX, MODE, false, false>), grid, block, smem, stream, args);
}

template <int E, int NWMAX>
hipError_t launch_mode(const LaunchArgs& args, int mode, int64_t n_blocks, hipStream_t stream) {
  const int nw = (NWMAX == 1) ? 1 : args.nw;
  // the bin area also holds the sampling weights of 5-16-wave rows while they seed
  const size_t smem = kSmemHdr + ((mode == MODE_FULL || mode == MODE_STEP || mode == MODE_SEED)
                                      ? kTableBytes + static_cast<size_t>(nw) * kBinBytesPerWave
                                      : 0);
  const dim3 grid(static_cast<unsigned>(n_blocks));
  const dim3 block(kWave * nw);
  const bool wide = args.group >= E;
  const bool var = args.variant != 0 || args.restart != 0;
  switch (mode) {
    case MODE_FULL: launch_kernel<E, NWMAX, MODE_FULL>(args, grid, block, smem, stream, wide, var); break;
    case MODE_SCALE: launch_kernel<E, NWMAX, MODE_SCALE>(args, grid, block, smem, stream, wide, var); break;
    case MODE_SEED: launch_kernel<E, NWMAX, MODE_SEED>(args, grid, block, smem, stream, wide, var); break;
    case MODE_STEP: launch_kernel<E, NWMAX, MODE_STEP>(args, grid, block, smem, stream, wide, var); break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace
}  // namespace any4
