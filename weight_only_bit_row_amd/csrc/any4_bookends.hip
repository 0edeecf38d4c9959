// Bookends of the any4 quantizer on gfx950 ("any4: Learned 4-bit Numeric
// Representation for LLMs", arXiv 2507.04610):
//   * E|x_j|, the per-channel mean absolute activation of a calibration batch that
//     the sample weights of Section 4.1 (Eq. 23) consume;
//   * dequantization of the emitted codes, Section 2.5.2 (Eq. 4):
//     w_hat = alpha * LUT[q] + beta.
// Both are streaming kernels bound by HBM bandwidth: every input byte is read once
// with 16-byte loads, every output byte written once, and nothing is re-read.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "any4_launch.h"

namespace any4 {
namespace {

constexpr int kThreads = 256;
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));   // 16-byte vectors for the
typedef float f32x4 __attribute__((ext_vector_type(4)));      // streaming loads and stores

// ---------------------------------------------------------------------------------
// E|x_j|.  Pass 1: workgroup (cx, s) covers 512 consecutive channels, 8 per lane, and
// token slice s; its four waves take every fourth token of the slice (wave w: tokens
// t0 + w, t0 + w + 4, ...), each summing |x| in fp64 in token order, and the four sums
// are added in wave order through LDS.  Pass 2: each channel's slice sums are added in
// slice order by four waves (a quarter of the slices each, combined in wave order),
// divided by T in fp64 and rounded to fp32.  The plan depends only on (T, K), so
// results are the same on every launch.

constexpr int kAbsChannels = 8;   // per lane: one 16-byte load of bf16, two of fp32
constexpr int kAbsUnroll = 16;    // tokens whose loads are in flight together per wave
constexpr int kAbsWaves = kThreads / 64;
constexpr int64_t kAbsBlockChannels = int64_t(64) * kAbsChannels;

__device__ __forceinline__ float bf16_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

__device__ __forceinline__ void add_abs8(double (&acc)[kAbsChannels], const u32x4& v, bool bf16,
                                         const u32x4& v2) {
  if (bf16) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += fabs(static_cast<double>(bf16_lo(w[i])));
      acc[2 * i + 1] += fabs(static_cast<double>(bf16_hi(w[i])));
    }
  } else {
    const uint32_t w[8] = {v.x, v.y, v.z, v.w, v2.x, v2.y, v2.z, v2.w};
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += fabs(static_cast<double>(__uint_as_float(w[i])));
  }
}

// VEC: K % 8 == 0 and x 16-byte aligned, so each lane's 8 channels of a token are one
// (bf16) or two (fp32) aligned 16-byte vectors.
template <bool BF16, bool VEC>
__global__ __launch_bounds__(kThreads) void absmean_partial_kernel(const void* __restrict__ x,
                                                                   int64_t T, int64_t K,
                                                                   int64_t tokens_per_split,
                                                                   double* __restrict__ partial) {
  __shared__ double red[kAbsWaves - 1][64][kAbsChannels];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j0 = (int64_t(blockIdx.x) * 64 + lane) * kAbsChannels;
  const int64_t s = blockIdx.y;
  const int64_t t0 = s * tokens_per_split;
  const int64_t t1 = (t0 + tokens_per_split < T) ? t0 + tokens_per_split : T;
  double acc[kAbsChannels];
#pragma unroll
  for (int i = 0; i < kAbsChannels; ++i) acc[i] = 0.0;
  if (j0 < K) {
    if (VEC) {
      constexpr int kElem = BF16 ? 2 : 4;
      const char* base = static_cast<const char*>(x) + j0 * kElem;
      const int64_t row_bytes = K * kElem;
      int64_t t = t0 + wave;
      for (; t + int64_t(kAbsWaves) * (kAbsUnroll - 1) < t1; t += int64_t(kAbsWaves) * kAbsUnroll) {
        u32x4 v[kAbsUnroll], v2[kAbsUnroll];
#pragma unroll
        for (int u = 0; u < kAbsUnroll; ++u) {
          const u32x4* p = reinterpret_cast<const u32x4*>(base + (t + kAbsWaves * u) * row_bytes);
          v[u] = __builtin_nontemporal_load(p);
          if (!BF16) v2[u] = __builtin_nontemporal_load(p + 1);
        }
#pragma unroll
        for (int u = 0; u < kAbsUnroll; ++u) add_abs8(acc, v[u], BF16, BF16 ? v[u] : v2[u]);
      }
      for (; t < t1; t += kAbsWaves) {
        const u32x4* p = reinterpret_cast<const u32x4*>(base + t * row_bytes);
        const u32x4 v = __builtin_nontemporal_load(p);
        const u32x4 v2 = BF16 ? v : __builtin_nontemporal_load(p + 1);
        add_abs8(acc, v, BF16, v2);
      }
    } else {
      for (int64_t t = t0 + wave; t < t1; t += kAbsWaves) {
#pragma unroll
        for (int i = 0; i < kAbsChannels; ++i) {
          const int64_t j = j0 + i;
          if (j < K) {
            float f;
            if (BF16)
              f = __uint_as_float(uint32_t(static_cast<const uint16_t*>(x)[t * K + j]) << 16);
            else
              f = static_cast<const float*>(x)[t * K + j];
            acc[i] += fabs(static_cast<double>(f));
          }
        }
      }
    }
  }
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < kAbsChannels; ++i) red[wave - 1][lane][i] = acc[i];
  }
  __syncthreads();
  if (wave == 0 && j0 < K) {
#pragma unroll
    for (int w = 0; w < kAbsWaves - 1; ++w)
#pragma unroll
      for (int i = 0; i < kAbsChannels; ++i) acc[i] += red[w][lane][i];
#pragma unroll
    for (int i = 0; i < kAbsChannels; ++i)
      if (j0 + i < K) partial[s * K + j0 + i] = acc[i];
  }
}

// 64 channels per workgroup; wave w adds slices w, w + 4, ... in order, then wave 0
// adds the four sums in wave order.
__global__ __launch_bounds__(kThreads) void absmean_finish_kernel(const double* __restrict__ partial,
                                                                  int64_t n_splits, int64_t T,
                                                                  int64_t K, float* __restrict__ out) {
  __shared__ double red[kAbsWaves - 1][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j = int64_t(blockIdx.x) * 64 + lane;
  double sum = 0.0;
  if (j < K) {
    int64_t s = wave;
    for (; s + 3 * kAbsWaves < n_splits; s += 4 * kAbsWaves) {  // four loads in flight
      const double p0 = partial[s * K + j], p1 = partial[(s + kAbsWaves) * K + j];
      const double p2 = partial[(s + 2 * kAbsWaves) * K + j], p3 = partial[(s + 3 * kAbsWaves) * K + j];
      sum += p0;
      sum += p1;
      sum += p2;
      sum += p3;
    }
    for (; s < n_splits; s += kAbsWaves) sum += partial[s * K + j];
  }
  if (wave > 0) red[wave - 1][lane] = sum;
  __syncthreads();
  if (wave == 0 && j < K) {
#pragma unroll
    for (int w = 0; w < kAbsWaves - 1; ++w) sum += red[w][lane];
    out[j] = static_cast<float>(sum / static_cast<double>(T));
  }
}

// ---------------------------------------------------------------------------------
// Dequantization.  A row's LUT is widened to fp32 in LDS (entries beyond n_clusters
// hold NaN, so a code outside the LUT gives NaN).  In the vector path each lane takes
// 8 consecutive columns at a time: one 4-byte load of codes (the 8 nibbles in column
// order, low nibble first), one alpha/beta pair (the group spans the 8 columns), and one
// 16-byte store of bf16 (two for fp32).  With bf16 output each store instruction of a
// wave then writes 1 KB contiguous, whole cache lines; 16 columns per lane step (two
// 16-byte stores, each covering half of every line) measured 10% slower on 14336 x 4096
// and 23% slower on 8192 x 28672, where the output does not stay in the last-level cache.

constexpr int kDqCols = 8;

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return static_cast<float>(v);  // exact widening
}

// two floats -> two bfloat16 in one register (low half first), round to nearest even,
// NaN stays NaN (gfx950 converts a pair in one instruction)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// w_hat = fl(fl(alpha * level) + beta): the kernels are built without contraction
__device__ __forceinline__ float dequant_one(float alpha, float level, float beta) {
  const float prod = alpha * level;
  return prod + beta;
}

__device__ __forceinline__ void dequant_store_chunk(void* out, int64_t off, float alpha, float beta,
                                                uint64_t nib, const float* lut, bool bf16_out) {
  float w[kDqCols];
#pragma unroll
  for (int e = 0; e < kDqCols; ++e) w[e] = dequant_one(alpha, lut[(nib >> (4 * e)) & 0xF], beta);
  if (bf16_out) {
    uint32_t p[kDqCols / 2];
#pragma unroll
    for (int e = 0; e < kDqCols / 2; ++e) p[e] = bf16x2_rne_bits(w[2 * e], w[2 * e + 1]);
    u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(out) + off);
    dst[0] = u32x4{p[0], p[1], p[2], p[3]};
  } else {
    f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(out) + off);
#pragma unroll
    for (int v = 0; v < kDqCols / 4; ++v)
      dst[v] = f32x4{w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]};
  }
}

// Vector path (K % 8 == 0, group % 8 == 0, aligned pointers): a workgroup takes
// kDqRows rows; chunk id = r * (K / 8) + c is columns [8c, 8c + 8) of row r, and
// lane t takes ids t, t + 256, ...  The codes and scale/offset of a lane's first
// kDqPre chunks are requested before the LUTs are staged, so their latency overlaps
// the LUT loads and the barrier.
constexpr int kDqRows = 4;
constexpr int kDqPre = 4;

template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void dequant_vec_kernel(const DequantDesc d) {
  __shared__ float lut[kDqRows][16];
  const int tid = threadIdx.x;
  const int64_t r0 = int64_t(blockIdx.x) * kDqRows;
  const int nr = (d.n_rows - r0 < kDqRows) ? static_cast<int>(d.n_rows - r0) : kDqRows;
  const int64_t K = d.n_cols, G = K / d.group;
  const int cpr = static_cast<int>(K / kDqCols);   // chunks per row (K <= 2^31 columns)
  // lane's chunk (row rr, chunk c) for id = tid, tid + 256, ...: step c by 256 and
  // carry whole rows into rr
  int rr = tid / cpr, c = tid - (tid / cpr) * cpr;
  uint64_t nib[kDqPre];
  uint16_t ab[kDqPre], bb[kDqPre];
  int pr[kDqPre], pc[kDqPre];
#pragma unroll
  for (int p = 0; p < kDqPre; ++p) {
    pr[p] = rr;
    pc[p] = c;
    nib[p] = 0;
    ab[p] = bb[p] = 0;
    if (rr < nr) {
      const int64_t r = r0 + rr, c0 = int64_t(c) * kDqCols;
      nib[p] = *reinterpret_cast<const uint32_t*>(d.codes + r * (K / 2) + c0 / 2);
      ab[p] = d.scale[r * G + c0 / d.group];
      bb[p] = d.offset[r * G + c0 / d.group];
    }
    c += kThreads;
    while (c >= cpr) {
      c -= cpr;
      ++rr;
    }
  }
  if (tid < nr * 16) {
    const int r = tid >> 4, e = tid & 15;
    lut[r][e] = e < d.n_clusters ? half_bits_to_float(d.lut[(r0 + r) * d.n_clusters + e])
                                 : __builtin_nanf("");
  }
  __syncthreads();
#pragma unroll
  for (int p = 0; p < kDqPre; ++p) {
    if (pr[p] < nr)
      dequant_store_chunk(d.out, (r0 + pr[p]) * K + int64_t(pc[p]) * kDqCols, half_bits_to_float(ab[p]),
                      half_bits_to_float(bb[p]), nib[p], lut[pr[p]], BF16_OUT);
  }
  for (; rr < nr;) {
    const int64_t r = r0 + rr, c0 = int64_t(c) * kDqCols;
    const uint64_t nb = *reinterpret_cast<const uint32_t*>(d.codes + r * (K / 2) + c0 / 2);
    dequant_store_chunk(d.out, r * K + c0, half_bits_to_float(d.scale[r * G + c0 / d.group]),
                    half_bits_to_float(d.offset[r * G + c0 / d.group]), nb, lut[rr], BF16_OUT);
    c += kThreads;
    while (c >= cpr) {
      c -= cpr;
      ++rr;
    }
  }
}

// Scalar path (any even K, any group): one workgroup per row, one column per lane step.
template <bool BF16_OUT>
__global__ __launch_bounds__(kThreads) void dequant_scalar_kernel(const DequantDesc d) {
  __shared__ float lut[16];
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t K = d.n_cols;
  const int64_t G = K / d.group;
  if (tid < 16)
    lut[tid] = tid < d.n_clusters ? half_bits_to_float(d.lut[row * d.n_clusters + tid])
                                  : __builtin_nanf("");
  __syncthreads();
  const uint8_t* codes = d.codes + row * (K / 2);
  const uint16_t* scale = d.scale + row * G;
  const uint16_t* offset = d.offset + row * G;
  for (int64_t j = tid; j < K; j += kThreads) {
    const uint8_t byte = codes[j / 2];
    const int q = (j & 1) ? (byte >> 4) : (byte & 0xF);
    const int64_t g = j / d.group;
    const float w = dequant_one(half_bits_to_float(scale[g]), lut[q], half_bits_to_float(offset[g]));
    if (BF16_OUT)
      static_cast<uint16_t*>(d.out)[row * K + j] = static_cast<uint16_t>(bf16x2_rne_bits(w, 0.0f));
    else
      static_cast<float*>(d.out)[row * K + j] = w;
  }
}

// ---------------------------------------------------------------------------------
// LUT-dequantized matrix-vector product for a few tokens (M <= 8), the consumer of the
// emitted format (the paper's tinygemm dequantizes on the fly before its multiply):
//   y[m][n] = sum_j x[m][j] * (alpha_{n,g(j)} * LUT_n[q_{n,j}] + beta_{n,g(j)}),
// taken per 16-column chunk c of one group as alpha * (sum_{j in c} x_j L_{q_j}) +
// beta * (sum_{j in c} x_j), all in fp32.  Its roofline is HBM at decode sizes: the codes
// are the only large operand (half a byte per weight); x is a few KB that every wave
// reads through L1/L2.
//
// One wave owns R rows (2 on rows up to 16384 columns, else 4) and one K-slice.  Lane l
// takes the 16-column chunks l, l + 64, ... of the slice for all R rows, so each 8-byte
// code load is part of a 512-byte contiguous run per row and each x value, converted
// once, serves R rows.  The row LUTs sit in LDS, 16 floats per row; a nibble's LDS
// address is formed by one byte permute that drops 4*q (shifted and masked, four nibbles
// per register) into byte 0 of the wave's 256-byte LUT block (the row offset is an
// immediate).  All lanes of a wave look up the same row at a time: 16 consecutive words,
// no bank conflicts.  With two or more tokens each row's LUT is first expanded into a
// 256-entry table indexed by a whole code byte (both of its elements' values, 8 bytes):
// half the LDS reads and no nibble unpacking, at the cost of bank conflicts, which
// measured 2-7% faster there and up to 6% slower at one token.  Partial sums of the R*MT
// outputs are reduced across the wave by a butterfly that halves the values held per
// lane at each step, and across the K-slices of a row group through LDS, in a fixed
// order (the result does not depend on timing).
constexpr int kGvWaves = 4;    // waves per workgroup

template <int N>
__device__ __forceinline__ float wave_reduce_spread(float (&v)[N], int lane) {
  // On return, lanes whose low (6 - log2 N) bits are zero hold the wave total of value
  // index lane >> (6 - log2 N).
  static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "N must be a power of two <= 64");
  int o = 32;
#pragma unroll
  for (int h = N / 2; h >= 1; h /= 2, o /= 2) {
    const bool up = (lane & o) != 0;
#pragma unroll
    for (int i = 0; i < h; ++i) {
      const float send = up ? v[i] : v[i + h];
      const float keep = up ? v[i + h] : v[i];
      v[i] = keep + __shfl_xor(send, o);
    }
  }
  float t = v[0];
  for (; o >= 1; o /= 2) t += __shfl_xor(t, o);
  return t;
}

__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t u) {
  bf16x2 v;
  __builtin_memcpy(&v, &u, 4);
  return v;
}

// One chunk's weight data for the wave's R rows: codes, and the alpha/beta bits of the
// chunk's group.
template <int R>
struct GvW {
  uint2 cw[R];
  uint16_t a[R], b[R];
};

// One chunk of x (16 columns of every token) as raw words, for prefetching.
template <int MT, bool XBF>
struct GvX {
  uint32_t w[MT][XBF ? 8 : 16];
};

template <int MT, bool XBF>
__device__ __forceinline__ void gv_load_x_raw(const GemvDesc& d, uint32_t col, GvX<MT, XBF>& x) {
#pragma unroll
  for (int m = 0; m < MT; ++m) {
    const int64_t base = (m < d.n_tokens ? m : d.n_tokens - 1) * d.n_cols;
    const u32x4* p = XBF ? reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(d.x) + base + col)
                         : reinterpret_cast<const u32x4*>(static_cast<const float*>(d.x) + base + col);
#pragma unroll
    for (int i = 0; i < (XBF ? 2 : 4); ++i) {
      const u32x4 v = p[i];
      x.w[m][4 * i] = v.x; x.w[m][4 * i + 1] = v.y; x.w[m][4 * i + 2] = v.z; x.w[m][4 * i + 3] = v.w;
    }
  }
}

// Rows per wave (R), chosen by row length.  Up to K = 16384 ("short rows") a wave takes 2
// rows: more waves hide more of the LUT-read and load latency (one token: 5% faster on
// 14336 x 4096; eight tokens: 30% faster, where the four-row instance needs ~230 VGPRs).
// Longer rows take 4, which converts each x value for more rows (one token, 8192 x 28672:
// 9% faster than two rows).  Eight rows per wave halve the wave count and were slower
// everywhere.
constexpr int kGvLongK = 16384;

template <int MT, bool XBF, int R>
__global__ __launch_bounds__(kThreads) void gemv_kernel(const GemvDesc d, int split_log2) {
  constexpr int XW = MT <= 2 ? 8 : 4;   // x columns converted per step (register budget)
  constexpr bool PX = MT <= 2;          // x of the next chunk prefetched with its codes (else
                                        // this chunk's x is loaded with the next codes)
  constexpr int RB = R < 4 ? 4 : R;     // LUT rows per wave block (at least 256 bytes)
  __shared__ __attribute__((aligned(1024))) float lut[kGvWaves][RB][16];
  // two or more tokens: a per-row table indexed by a whole code byte holding both of its
  // elements' LUT values, one 8-byte LDS read per two weights
  constexpr bool PT = MT >= 2;
  __shared__ __attribute__((aligned(16))) float2 ptab[PT ? kGvWaves : 1][PT ? R : 1][PT ? 256 : 1];
  __shared__ float part[kGvWaves][R * MT];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int splits = 1 << split_log2;
  const int ks = wave & (splits - 1);
  const int64_t row0 =
      ((int64_t(blockIdx.x) << (2 - split_log2)) + (wave >> split_log2)) * R;  // 4 waves per WG
  const int64_t N = d.n_rows, K = d.n_cols;
  const int gshift = __builtin_ctz(static_cast<uint32_t>(d.group));
  const int64_t G = K >> gshift;
  // the wave's LUT entries (16 per row) are fetched first and stored below
  static_assert(RB % 4 == 0, "LUT rows of 16 entries are loaded 64 at a time");
  uint16_t lut_bits[RB / 4];
#pragma unroll
  for (int i = 0; i < RB / 4; ++i) {
    const int r = (lane >> 4) + 4 * i, q = lane & 15;
    const bool ok = r < R && row0 + r < N && q < d.n_clusters;
    lut_bits[i] = d.lut[ok ? (row0 + r) * d.n_clusters + q : 0];  // no branch
  }
  const uint8_t* codes[R];
  const char* scale[R];
  const char* offset[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = (row0 + r < N) ? row0 + r : N - 1;  // tail rows: read row N-1, never stored
    codes[r] = d.codes + row * (K >> 1);
    scale[r] = reinterpret_cast<const char*>(d.scale + row * G);
    offset[r] = reinterpret_cast<const char*>(d.offset + row * G);
  }
  const uint32_t chunks = static_cast<uint32_t>(K >> 4);
  const uint32_t per = (chunks + splits - 1) >> split_log2;
  const uint32_t c_begin = ks * per;
  const uint32_t c_end = c_begin + per < chunks ? c_begin + per : chunks;
  const uint32_t c_last = c_end > c_begin ? c_end - 1 : c_begin;  // clamp for prefetches
  auto load_w = [&](GvW<R>& w, uint32_t c) {
    const uint32_t gb = ((c << 4) >> gshift) << 1;  // byte offset of the group's alpha/beta
#pragma unroll
    for (int r = 0; r < R; ++r) {
      w.cw[r] = *reinterpret_cast<const uint2*>(codes[r] + (c << 3));
      w.a[r] = *reinterpret_cast<const uint16_t*>(scale[r] + gb);
      w.b[r] = *reinterpret_cast<const uint16_t*>(offset[r] + gb);
    }
  };
  uint32_t c = c_begin + lane;
  GvW<R> wcur;
  GvX<MT, XBF> xcur;
  load_w(wcur, c < c_last ? c : c_last);
  if constexpr (PX) gv_load_x_raw<MT, XBF>(d, (c < c_last ? c : c_last) << 4, xcur);
#pragma unroll
  for (int i = 0; i < RB / 4; ++i) {
    const int r = (lane >> 4) + 4 * i, q = lane & 15;
    lut[wave][r][q] = (r < R && row0 + r < N && q < d.n_clusters) ? half_bits_to_float(lut_bits[i])
                                                                   : __builtin_nanf("");
  }
  // each wave reads only its own LUT block; LDS operations of a wave complete in order
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  if constexpr (PT) {
    // entry b of row r: (LUT[b & 15], LUT[b >> 4]), the low nibble being the even column
    for (int i = lane; i < 256 * R; i += 64) {
      const int r = i >> 8, b = i & 255;
      ptab[wave][r][b] = make_float2(lut[wave][r][b & 15], lut[wave][r][b >> 4]);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  // byte 0 of a LUT address comes from the codes, bytes 1..3 from the wave's block
  const uint32_t block = static_cast<uint32_t>(wave) * (RB * 64u);
  const char* lut_bytes = reinterpret_cast<const char*>(&lut[0][0][0]);
  float y[R][MT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) y[r][m] = 0.0f;

  for (; c < c_end; c += 64) {
    const uint32_t cn = c + 64 < c_last ? c + 64 : c_last;
    GvW<R> wnext;
    GvX<MT, XBF> xnext;
    load_w(wnext, cn);
    if constexpr (PX)
      gv_load_x_raw<MT, XBF>(d, cn << 4, xnext);
    else
      gv_load_x_raw<MT, XBF>(d, c << 4, xcur);  // this chunk's x, issued with the next codes
    __builtin_amdgcn_sched_barrier(0);  // the next chunk's loads go out before this one's math
    float acc[R][MT], xs[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) {
      xs[m] = 0.0f;
#pragma unroll
      for (int r = 0; r < R; ++r) acc[r][m] = 0.0f;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // the two 8-nibble words of the chunk
      uint32_t wr[R], lo4[R], hi4[R];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        wr[r] = h ? wcur.cw[r].y : wcur.cw[r].x;
        if constexpr (!PT) {
          lo4[r] = (wr[r] << 2) & 0x3C3C3C3Cu;   // 4 * nibbles 0, 2, 4, 6
          hi4[r] = (wr[r] >> 2) & 0x3C3C3C3Cu;   // 4 * nibbles 1, 3, 5, 7
        }
      }
#pragma unroll
      for (int qq = 0; qq < 8 / XW; ++qq) {  // XW columns of x at a time
        const int e0 = 8 * h + XW * qq;      // first column of this step within the chunk
        float xv[MT][XW];
#pragma unroll
        for (int m = 0; m < MT; ++m)
#pragma unroll
          for (int e = 0; e < XW; ++e) {
            const int j = e0 + e;
            xv[m][e] = XBF ? ((j & 1) ? bf16_hi(xcur.w[m][j >> 1]) : bf16_lo(xcur.w[m][j >> 1]))
                           : __uint_as_float(xcur.w[m][j]);
          }
        if constexpr (XBF) {
          // sum of a bf16 pair in one dot product with (1, 1): exact products, fp32 sum
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int e = 0; e < XW; e += 2)
              xs[m] = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(xcur.w[m][(e0 + e) >> 1]),
                                                      as_bf16x2(0x3F803F80u), xs[m], false);
        } else {
#pragma unroll
          for (int m = 0; m < MT; ++m)
#pragma unroll
            for (int e = 0; e < XW; ++e) xs[m] += xv[m][e];
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
#pragma unroll
          for (int jj = 0; jj < XW / 2; ++jj) {
            const int jb = jj + (XW / 2) * qq;  // code byte within the word
            float le, lo;
            if constexpr (PT) {
              const float2 L = ptab[wave][r][(wr[r] >> (8 * jb)) & 0xFFu];
              le = L.x;
              lo = L.y;
            } else {
              const uint32_t sel = 0x07060500u | uint32_t(jb);
              le = *reinterpret_cast<const float*>(
                  lut_bytes + __builtin_amdgcn_perm(block, lo4[r], sel) + r * 64);
              lo = *reinterpret_cast<const float*>(
                  lut_bytes + __builtin_amdgcn_perm(block, hi4[r], sel) + r * 64);
            }
#pragma unroll
            for (int m = 0; m < MT; ++m) {
              acc[r][m] = fmaf(xv[m][2 * jj], le, acc[r][m]);
              acc[r][m] = fmaf(xv[m][2 * jj + 1], lo, acc[r][m]);
            }
          }
        }
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      // fp16 alpha/beta feed mixed-precision multiply-adds (exact widening)
      const float al = half_bits_to_float(wcur.a[r]), be = half_bits_to_float(wcur.b[r]);
#pragma unroll
      for (int m = 0; m < MT; ++m) y[r][m] = fmaf(be, xs[m], fmaf(al, acc[r][m], y[r][m]));
    }
    wcur = wnext;
    if constexpr (PX) xcur = xnext;
  }

  constexpr int NV = R * MT;
  constexpr int kLow = (NV >= 64) ? 1 : 64 / NV;  // lanes per reduced value
  float v[NV];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int m = 0; m < MT; ++m) v[r * MT + m] = y[r][m];
  const float t = wave_reduce_spread<NV>(v, lane);
  const int idx = lane / kLow;
  const bool holder = (lane % kLow) == 0;
  if (splits > 1) {
    if (holder) part[wave][idx] = t;
    __syncthreads();
    if (ks != 0 || lane >= NV) return;
    float s = part[wave][lane];
    for (int k = 1; k < splits; ++k) s += part[wave + k][lane];
    const int r = lane / MT, m = lane % MT;
    if (row0 + r < N && m < d.n_tokens) d.y[m * N + row0 + r] = s;
  } else if (holder) {
    const int r = idx / MT, m = idx % MT;
    if (row0 + r < N && m < d.n_tokens) d.y[m * N + row0 + r] = t;
  }
}

// ---------------------------------------------------------------------------------
// The LUT product on the matrix cores, for bf16 activations and groups a multiple of 32
// columns.  With Eq. 4's w_hat = alpha * L[q] + beta, the columns j of one block (inside
// one group g) of row i give
//   sum_j x[t][j] * w_hat[i][j] = alpha_ig * sum_j x[t][j] L_i[q_ij] + beta_ig * sum_j x[t][j].
// The row's fp16 LUT values are split exactly into two bf16 parts, L = Lh + Ll (an fp16
// value has 11 significant bits, bf16 8, so the remainder needs at most 4), and the sums
// come from v_mfma_f32_16x16x32_bf16: products of bf16 values are exact in fp32 and
// accumulate in fp32, the arithmetic of the VALU kernel up to the summation order.
//
// The reduction index k of the L sums runs over (column, part) pairs: operand B holds
// (Lh, Ll) of a column in two neighbouring k slots, which is one lookup of a table entry
// stored as Lh | Ll << 16, and operand A holds that column's x twice.  So one MFMA covers
// 16 columns, lane l holding 4 of them:
//   A (16 x 32, bf16): token t = l % 16, (x_c, x_c) for each of the lane's columns c (rows
//       t >= n_tokens repeat the last token: their outputs are not stored)
//   B (32 x 16, bf16): row i = l % 16's (Lh, Ll) at those columns' codes
//   C (16 x 16, fp32): lane l holds tokens 4 (l / 16) + r, r < 4, of row l % 16
// and the x sums take one more MFMA per 32 columns with x in plain order against ones.
// Per block, y[t][i] += alpha_ig * C_L + beta_ig * C_S in fp32.
//
// A workgroup takes two tiles of 16 rows, and its W waves (W = 2, 4 or 8, by row length)
// split the row's blocks of 32 NMF columns (NMF = 1, 2, 4 for groups of 32, 64 and 128 or
// more) into W contiguous ranges; the W partial results are added in LDS in wave order (a
// fixed order, so repeated calls give the same bits).  In a block, lane l holds row
// i = l % 16 of each tile and the 8 NMF consecutive columns that lane group h = l / 16
// owns.  The x operand and the x sums serve both tiles.  All loads are buffer loads with
// per-lane offsets fixed for the whole call and the block's offset in a scalar register.
// The alpha/beta pairs are loaded once per four blocks (lane group h holds block h's pair
// for its rows) and reach the other lanes through ds_bpermute.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float mf32x4_t __attribute__((ext_vector_type(4)));
constexpr int kMfTiles = 2;                  // 16-row tiles per workgroup
constexpr int kMfRows = 16 * kMfTiles;       // rows per workgroup
constexpr int64_t kMfMaxCols = int64_t(1) << 26;   // per-lane buffer offsets stay 32-bit
constexpr int kRawBufferWord3 = 0x00020000;  // raw buffer resource word 3 on gfx9 parts

__device__ __forceinline__ bf16x8_t as_bf16x8(const u32x4& v) {
  bf16x8_t r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}

// fp32 -> bf16 bits, round to nearest even (finite values; NaN stays NaN)
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7F800000u) == 0x7F800000u) return (u >> 16) | ((u & 0x7FFFFFu) ? 0x40u : 0u);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint64_t bytes) {
  const uint64_t n = bytes < 0xFFFFFFFFull ? bytes : 0xFFFFFFFFull;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, static_cast<int>(n),
                                           kRawBufferWord3);
}

// Each lane's data for one block of 32 * NMF columns: its codes in each tile (NMF 4-byte
// words) and its token's x (NMF 16-byte vectors).
template <int NMF>
struct MfBlock {
  uint32_t w[kMfTiles][NMF];
  u32x4 x[NMF];
};

template <int NMF, int NW>
__global__ __launch_bounds__(NW * 64) void gemv_mfma_kernel(const GemvDesc d) {
  constexpr int BC = 32 * NMF;   // columns per block; lane group h takes BC / 4 of them
  // Lane l's LUT entry q, for row l % 16 of tile T, at word (16 T + q) * 64 + l: Lh bits |
  // Ll bits << 16 (a code past the LUT: Lh NaN, Ll 0).  A lane only reads its own column,
  // so every read of a wave hits 64 distinct banks whatever the codes (no bank
  // conflicts); all waves map lanes to rows the same way and share the table.
  __shared__ __attribute__((aligned(1024))) uint32_t ltab[kMfTiles][16][64];
  __shared__ mf32x4_t part[NW][kMfTiles][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t N = d.n_rows, K = d.n_cols;
  const int64_t row0 = int64_t(blockIdx.x) * kMfRows;
  const int64_t n_blocks = K / BC;
  const int64_t per = (n_blocks + NW - 1) / NW;
  const int64_t b_begin = wave * per < n_blocks ? wave * per : n_blocks;
  const int64_t b_end = b_begin + per < n_blocks ? b_begin + per : n_blocks;
  // every load is unconditional, its block clamped to the wave's range (a wave with no
  // blocks reads the row's last one): loads under a branch make the compiler wait for
  // every load in flight where the branches join
  const int64_t b_last = b_end > b_begin ? b_end - 1 : n_blocks - 1;
  const int i = lane & 15, h = lane >> 4;
  // this lane's token in operand A; rows of A past the last token repeat it (their outputs
  // are never stored), so every lane loads without a branch
  const int t = (lane & 15) < d.n_tokens ? (lane & 15) : static_cast<int>(d.n_tokens) - 1;
  const int gshift = __builtin_ctz(static_cast<uint32_t>(d.group));
  const int64_t n_groups = K >> gshift;
  // buffers based at the workgroup's first row; tail rows read row N - 1, never stored
  const uint32_t half_k = static_cast<uint32_t>(K >> 1);
  const __amdgpu_buffer_rsrc_t rc = buffer_rsrc(d.codes + row0 * (K >> 1), uint64_t(N - row0) * half_k);
  const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(d.scale + row0 * n_groups, uint64_t(N - row0) * n_groups * 2);
  const __amdgpu_buffer_rsrc_t ro = buffer_rsrc(d.offset + row0 * n_groups, uint64_t(N - row0) * n_groups * 2);
  const __amdgpu_buffer_rsrc_t rx = buffer_rsrc(d.x, uint64_t(d.n_tokens) * K * 2);
  uint32_t voff_c[kMfTiles], voff_p[kMfTiles];
#pragma unroll
  for (int T = 0; T < kMfTiles; ++T) {
    const int64_t r = row0 + 16 * T + i;
    const uint32_t rr = static_cast<uint32_t>((r < N ? r : N - 1) - row0);
    voff_c[T] = rr * half_k + (BC / 8) * h;
    voff_p[T] = rr * static_cast<uint32_t>(n_groups) * 2;
  }
  const uint32_t voff_x = static_cast<uint32_t>(t) * static_cast<uint32_t>(K) * 2 + (BC / 4) * h * 2;
  auto load = [&](MfBlock<NMF>& m, int64_t b) {
    const int bc = static_cast<int>(b) * (BC / 2);   // the block's byte offset in a code row
#pragma unroll
    for (int T = 0; T < kMfTiles; ++T) {
      if constexpr (NMF == 4) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rc, voff_c[T], bc, 0);
        m.w[T][0] = v.x; m.w[T][1] = v.y; m.w[T][2] = v.z; m.w[T][3] = v.w;
      } else {
#pragma unroll
        for (int s = 0; s < NMF; ++s) m.w[T][s] = __builtin_amdgcn_raw_buffer_load_b32(rc, voff_c[T] + 4 * s, bc, 0);
      }
    }
#pragma unroll
    for (int s = 0; s < NMF; ++s) m.x[s] = __builtin_amdgcn_raw_buffer_load_b128(rx, voff_x + 16 * s, 4 * bc, 0);
  };
  // alpha | beta << 16 of block b0 + h (clamped) for this lane's rows
  auto load_params = [&](uint32_t (&p)[kMfTiles], int64_t b0) {
    const int64_t b = b0 + h < b_last ? b0 + h : b_last;
    const uint32_t g2 = ((static_cast<uint32_t>(b) * BC) >> gshift) * 2;
#pragma unroll
    for (int T = 0; T < kMfTiles; ++T) {
      const uint32_t a = __builtin_amdgcn_raw_buffer_load_b16(rs, voff_p[T] + g2, 0, 0);
      const uint32_t o = __builtin_amdgcn_raw_buffer_load_b16(ro, voff_p[T] + g2, 0, 0);
      p[T] = (a & 0xFFFFu) | (o << 16);
    }
  };
  // the tables' 2048 words, 2048 / (64 NW) per thread, loaded first; then the first
  // blocks' loads go out, so that the wait for the LUT words does not wait for them
  constexpr int kPer = kMfTiles * 16 * 64 / (NW * 64);
  uint16_t lbits[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int n = tid + u * NW * 64;
    const int T = n >> 10, q = (n >> 6) & 15, ti = n & 15;
    const int64_t r = row0 + 16 * T + ti;
    const int64_t trow = r < N ? r : N - 1;
    lbits[u] = d.lut[trow * d.n_clusters + (q < d.n_clusters ? q : 0)];
  }
  // (the first pairs before the first blocks: the loop's first wait is for the pairs)
  auto clampb = [&](int64_t b) { return b < b_last ? b : b_last; };
  MfBlock<NMF> b0, b1, b2, b3;
  uint32_t pc[kMfTiles], pn[kMfTiles];
  load_params(pn, b_begin);
  load(b0, clampb(b_begin));
  load(b1, clampb(b_begin + 1));
  load(b2, clampb(b_begin + 2));
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int n = tid + u * NW * 64;
    const int T = n >> 10, q = (n >> 6) & 15;
    // computed for every entry and then selected, so that no load is sunk into a branch
    const float L = half_bits_to_float(lbits[u]);
    const uint32_t hb = bf16_rne_bits(L);
    const float lo = L - __uint_as_float(hb << 16);   // exact: at most 4 significant bits
    const uint32_t e = hb | ((__float_as_uint(lo) >> 16) << 16);
    ltab[T][q][n & 63] = q < d.n_clusters ? e : 0x7FC0u;   // past the LUT: NaN, 0
  }
  __syncthreads();                                       // the LUT tables are ready
  // byte address of entry q of this lane in tile 0: q << 8 | 4 lane, byte 1 from a nibble,
  // byte 0 the lane's column (one v_perm per lookup); tile T adds T * 4096
  const uint32_t lane4 = 4u * static_cast<uint32_t>(lane);
  const char* tbytes = reinterpret_cast<const char*>(&ltab[0][0][0]);
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  mf32x4_t y[kMfTiles];
#pragma unroll
  for (int T = 0; T < kMfTiles; ++T) y[T] = mf32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
  // one block (j-th of its group of four): every table lookup of the block first, then
  // the MFMA chains (per tile x * (Lh, Ll), once x * 1), then y += alpha C_L + beta C_S
  auto compute = [&](const MfBlock<NMF>& cur, int j, bool valid) {
    uint32_t g[kMfTiles][8 * NMF];     // entry of column c of the lane's 8 NMF
#pragma unroll
    for (int T = 0; T < kMfTiles; ++T) {
      const char* tb = tbytes + T * 4096;
#pragma unroll
      for (int s = 0; s < NMF; ++s) {
        const uint32_t w = cur.w[T][s];
        const uint32_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;  // nibbles 2p, 2p + 1
#pragma unroll
        for (int p = 0; p < 4; ++p) {                 // code byte p: columns 2p and 2p + 1
          const uint32_t sel = 0x0C0C0000u | ((4u + p) << 8);
          g[T][8 * s + 2 * p] = *reinterpret_cast<const uint32_t*>(tb + __builtin_amdgcn_perm(lo, lane4, sel));
          g[T][8 * s + 2 * p + 1] = *reinterpret_cast<const uint32_t*>(tb + __builtin_amdgcn_perm(hi, lane4, sel));
        }
      }
    }
    mf32x4_t cs = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s = 0; s < NMF; ++s)
      cs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(cur.x[s]), as_bf16x8(ones), cs, 0, 0, 0);
    mf32x4_t cl[kMfTiles];
#pragma unroll
    for (int T = 0; T < kMfTiles; ++T) cl[T] = mf32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int u = 0; u < 2 * NMF; ++u) {     // columns 4u .. 4u + 3 of the lane's 8 NMF
      const u32x4& xs = cur.x[u >> 1];
      const uint32_t x0 = (u & 1) ? xs.z : xs.x, x1 = (u & 1) ? xs.w : xs.y;
      // (x_c, x_c) for each column: the low or the high bf16 of an x word, twice
      const u32x4 a = {__builtin_amdgcn_perm(x0, x0, 0x01000100u), __builtin_amdgcn_perm(x0, x0, 0x03020302u),
                       __builtin_amdgcn_perm(x1, x1, 0x01000100u), __builtin_amdgcn_perm(x1, x1, 0x03020302u)};
#pragma unroll
      for (int T = 0; T < kMfTiles; ++T) {
        const u32x4 bv = {g[T][4 * u], g[T][4 * u + 1], g[T][4 * u + 2], g[T][4 * u + 3]};
        cl[T] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(bv), cl[T], 0, 0, 0);
      }
    }
#pragma unroll
    for (int T = 0; T < kMfTiles; ++T) {
      // this block's pair sits in lane i + 16 j
      const uint32_t ab = static_cast<uint32_t>(
          __builtin_amdgcn_ds_bpermute(4 * (i + 16 * j), static_cast<int>(pc[T])));
      const float al = half_bits_to_float(static_cast<uint16_t>(ab));
      const float be = half_bits_to_float(static_cast<uint16_t>(ab >> 16));
      if (valid) {
#pragma unroll
        for (int r = 0; r < 4; ++r) y[T][r] = fmaf(be, cs[r], fmaf(al, cl[T][r], y[T][r]));
      }
    }
  };
  // Four buffers in rotation, loads three blocks ahead.  The rotation is unrolled rather
  // than copied: a copy of a buffer whose loads are in flight would wait for them.
  // A group of four always runs all four steps (the loads stay unconditional); a block
  // past the wave's range adds nothing.
  auto step = [&](const MfBlock<NMF>& cur, MfBlock<NMF>& fill, int64_t b, int j) {
    load(fill, clampb(b + 3));
    __builtin_amdgcn_sched_barrier(0);  // the later block's loads go out before this one's math
    compute(cur, j, b < b_end);
  };
  for (int64_t b = b_begin; b < b_end; b += 4) {
#pragma unroll
    for (int T = 0; T < kMfTiles; ++T) pc[T] = pn[T];
    load_params(pn, b + 4);
    step(b0, b3, b, 0);
    step(b1, b0, b + 1, 1);
    step(b2, b1, b + 2, 2);
    step(b3, b2, b + 3, 3);
  }
#pragma unroll
  for (int T = 0; T < kMfTiles; ++T) part[wave][T][lane] = y[T];
  __syncthreads();
  if (wave >= kMfTiles) return;
  // wave T adds tile T's partial results in wave order
  mf32x4_t acc = part[0][wave][lane];
  for (int w = 1; w < NW; ++w) {
    const mf32x4_t v = part[w][wave][lane];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] += v[r];
  }
  // lane l holds tokens 4 (l / 16) + r of row l % 16 of the tile
  const int64_t orow = row0 + 16 * wave + i;
  if (orow < N) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = 4 * h + r;
      if (tok < d.n_tokens) d.y[int64_t(tok) * N + orow] = acc[r];
    }
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

AbsmeanPlan plan_absmean(int64_t n_tokens, int64_t n_cols) {
  // about 1024 workgroups (4 per CU) and at least 256 tokens (64 per wave) per slice
  const int64_t col_blocks = (n_cols + kAbsBlockChannels - 1) / kAbsBlockChannels;
  int64_t splits = (1024 + col_blocks - 1) / col_blocks;
  const int64_t max_splits = (n_tokens + 255) / 256;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  if (splits > 65535) splits = 65535;
  AbsmeanPlan p;
  p.tokens_per_split = (n_tokens + splits - 1) / splits;
  p.n_splits = (n_tokens + p.tokens_per_split - 1) / p.tokens_per_split;
  p.partial_bytes = size_t(p.n_splits) * size_t(n_cols) * sizeof(double);
  return p;
}

hipError_t launch_absmean(const void* x, int dtype, int64_t n_tokens, int64_t n_cols, float* out,
                          double* partial, const AbsmeanPlan& plan, hipStream_t stream) {
  const bool bf16 = dtype == 1;
  const bool vec = (n_cols % kAbsChannels == 0) && aligned(x, 16);
  const dim3 grid(static_cast<uint32_t>((n_cols + kAbsBlockChannels - 1) / kAbsBlockChannels),
                  static_cast<uint32_t>(plan.n_splits));
  if (bf16 && vec)
    hipLaunchKernelGGL((absmean_partial_kernel<true, true>), grid, dim3(kThreads), 0, stream, x,
                       n_tokens, n_cols, plan.tokens_per_split, partial);
  else if (bf16)
    hipLaunchKernelGGL((absmean_partial_kernel<true, false>), grid, dim3(kThreads), 0, stream, x,
                       n_tokens, n_cols, plan.tokens_per_split, partial);
  else if (vec)
    hipLaunchKernelGGL((absmean_partial_kernel<false, true>), grid, dim3(kThreads), 0, stream, x,
                       n_tokens, n_cols, plan.tokens_per_split, partial);
  else
    hipLaunchKernelGGL((absmean_partial_kernel<false, false>), grid, dim3(kThreads), 0, stream, x,
                       n_tokens, n_cols, plan.tokens_per_split, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(absmean_finish_kernel, dim3(static_cast<uint32_t>((n_cols + 63) / 64)),
                     dim3(kThreads), 0, stream, partial, plan.n_splits, n_tokens, n_cols, out);
  return hipGetLastError();
}

template <int NMF>
hipError_t launch_gemv_mfma(const GemvDesc& d, int nw, hipStream_t stream) {
  const dim3 grid(static_cast<uint32_t>((d.n_rows + kMfRows - 1) / kMfRows));
  if (nw == 8)
    hipLaunchKernelGGL((gemv_mfma_kernel<NMF, 8>), grid, dim3(8 * 64), 0, stream, d);
  else if (nw == 4)
    hipLaunchKernelGGL((gemv_mfma_kernel<NMF, 4>), grid, dim3(4 * 64), 0, stream, d);
  else
    hipLaunchKernelGGL((gemv_mfma_kernel<NMF, 2>), grid, dim3(2 * 64), 0, stream, d);
  return hipGetLastError();
}

int plan_gemv_split_log2(int64_t n_rows, int64_t n_cols, int rows_per_wave, int64_t target) {
  // split K over up to 4 waves of a workgroup while the grid holds fewer than `target`
  // waves and every lane keeps at least two chunks of its slice
  const int64_t groups = (n_rows + rows_per_wave - 1) / rows_per_wave, chunks = n_cols / 16;
  int l = 0;
  while ((1 << l) < kGvWaves && groups << l < target && chunks >> (l + 1) >= 128) ++l;
  return l;
}

template <int MT, int R>
hipError_t launch_gemv_mt(const GemvDesc& d, hipStream_t stream) {
  // up to four tokens: short waves whose LUT reads want latency hiding, 16 waves per CU;
  // eight tokens: 8 per CU (more registers per wave)
  const int l = plan_gemv_split_log2(d.n_rows, d.n_cols, R, MT <= 4 ? 4096 : 2048);
  const int64_t groups = (d.n_rows + R - 1) / R;
  const int64_t per_wg = kGvWaves >> l;
  const dim3 grid(static_cast<uint32_t>((groups + per_wg - 1) / per_wg));
  if (d.x_bf16)
    hipLaunchKernelGGL((gemv_kernel<MT, true, R>), grid, dim3(kThreads), 0, stream, d, l);
  else
    hipLaunchKernelGGL((gemv_kernel<MT, false, R>), grid, dim3(kThreads), 0, stream, d, l);
  return hipGetLastError();
}

hipError_t launch_gemv(const GemvDesc& d, hipStream_t stream) {
  if (d.n_rows == 0) return hipSuccess;
  // bf16 activations and groups of whole 32-column MFMA steps go to the matrix cores
  if (d.x_bf16 && d.group % 32 == 0 && d.n_tokens >= kGemvMfmaMinTokens && d.n_cols <= kMfMaxCols &&
      aligned(d.x, 16) && aligned(d.codes, 16)) {
    // waves per workgroup: at least 8 blocks of 128 columns per wave, at most 8 waves
    const int64_t kb = d.n_cols / 128;
    const int nw = kb >= 64 ? 8 : kb >= 32 ? 4 : 2;
    if (d.group == 32) return launch_gemv_mfma<1>(d, nw, stream);
    if (d.group == 64) return launch_gemv_mfma<2>(d, nw, stream);
    return launch_gemv_mfma<4>(d, nw, stream);
  }
  const bool short_rows = d.n_cols <= kGvLongK;
  if (d.n_tokens <= 1)
    return short_rows ? launch_gemv_mt<1, 2>(d, stream) : launch_gemv_mt<1, 4>(d, stream);
  if (d.n_tokens <= 2)
    return short_rows ? launch_gemv_mt<2, 2>(d, stream) : launch_gemv_mt<2, 4>(d, stream);
  if (d.n_tokens <= 4)
    return short_rows ? launch_gemv_mt<4, 2>(d, stream) : launch_gemv_mt<4, 4>(d, stream);
  return short_rows ? launch_gemv_mt<8, 2>(d, stream) : launch_gemv_mt<8, 4>(d, stream);
}

hipError_t launch_dequant(const DequantDesc& d, hipStream_t stream) {
  if (d.n_rows == 0) return hipSuccess;
  const bool vec = d.n_cols % kDqCols == 0 && d.group % kDqCols == 0 && aligned(d.codes, 8) &&
                   aligned(d.out, 16);
  const dim3 grid_vec(static_cast<uint32_t>((d.n_rows + kDqRows - 1) / kDqRows));
  const dim3 grid_row(static_cast<uint32_t>(d.n_rows));
  if (d.out_bf16 && vec)
    hipLaunchKernelGGL((dequant_vec_kernel<true>), grid_vec, dim3(kThreads), 0, stream, d);
  else if (d.out_bf16)
    hipLaunchKernelGGL((dequant_scalar_kernel<true>), grid_row, dim3(kThreads), 0, stream, d);
  else if (vec)
    hipLaunchKernelGGL((dequant_vec_kernel<false>), grid_vec, dim3(kThreads), 0, stream, d);
  else
    hipLaunchKernelGGL((dequant_scalar_kernel<false>), grid_row, dim3(kThreads), 0, stream, d);
  return hipGetLastError();
}

}  // namespace any4
