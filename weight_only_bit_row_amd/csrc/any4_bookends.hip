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
// E|x_j|.  Pass 1: block (cx, s) sums |x| over token slice s for 2048 consecutive
// channels, 8 per lane, in fp64 and in token order.  Pass 2: channel j sums the
// slices' partial sums in slice order, divides by T in fp64 and rounds to fp32.  The
// slice plan depends only on (T, K), so results are the same on every launch.

constexpr int kAbsChannels = 8;   // per lane: one 16-byte load of bf16, two of fp32
constexpr int kAbsUnroll = 8;     // tokens whose loads are in flight together
constexpr int64_t kAbsBlockChannels = int64_t(kThreads) * kAbsChannels;

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
  const int64_t j0 = (int64_t(blockIdx.x) * kThreads + threadIdx.x) * kAbsChannels;
  if (j0 >= K) return;
  const int64_t s = blockIdx.y;
  const int64_t t0 = s * tokens_per_split;
  const int64_t t1 = (t0 + tokens_per_split < T) ? t0 + tokens_per_split : T;
  double acc[kAbsChannels];
#pragma unroll
  for (int i = 0; i < kAbsChannels; ++i) acc[i] = 0.0;
  if (VEC) {
    // row t starts at element t*K; 16-byte vectors of this lane's channels
    constexpr int kElem = BF16 ? 2 : 4;
    const char* base = static_cast<const char*>(x) + j0 * kElem;
    const int64_t row_bytes = K * kElem;
    int64_t t = t0;
    for (; t + kAbsUnroll <= t1; t += kAbsUnroll) {
      u32x4 v[kAbsUnroll], v2[kAbsUnroll];
#pragma unroll
      for (int u = 0; u < kAbsUnroll; ++u) {
        const u32x4* p = reinterpret_cast<const u32x4*>(base + (t + u) * row_bytes);
        v[u] = __builtin_nontemporal_load(p);
        if (!BF16) v2[u] = __builtin_nontemporal_load(p + 1);
      }
#pragma unroll
      for (int u = 0; u < kAbsUnroll; ++u) add_abs8(acc, v[u], BF16, BF16 ? v[u] : v2[u]);
    }
    for (; t < t1; ++t) {
      const u32x4* p = reinterpret_cast<const u32x4*>(base + t * row_bytes);
      const u32x4 v = __builtin_nontemporal_load(p);
      const u32x4 v2 = BF16 ? v : __builtin_nontemporal_load(p + 1);
      add_abs8(acc, v, BF16, v2);
    }
  } else {
    for (int64_t t = t0; t < t1; ++t) {
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
#pragma unroll
  for (int i = 0; i < kAbsChannels; ++i)
    if (j0 + i < K) partial[s * K + j0 + i] = acc[i];
}

__global__ __launch_bounds__(kThreads) void absmean_finish_kernel(const double* __restrict__ partial,
                                                                  int64_t n_splits, int64_t T,
                                                                  int64_t K, float* __restrict__ out) {
  const int64_t j = int64_t(blockIdx.x) * kThreads + threadIdx.x;
  if (j >= K) return;
  double sum = 0.0;
  for (int64_t s = 0; s < n_splits; ++s) sum += partial[s * K + j];
  out[j] = static_cast<float>(sum / static_cast<double>(T));
}

// ---------------------------------------------------------------------------------
// Dequantization.  One workgroup per row; the row's LUT is widened to fp32 in LDS
// (entries beyond n_clusters hold NaN, so a code outside the LUT gives NaN).  In the
// vector path each lane takes 16 consecutive columns: one 8-byte load of codes (the
// 16 nibbles in column order, low nibble first), one alpha/beta pair when the group
// spans them, and 64 (fp32) or 32 (bf16) bytes of 16-byte stores.

constexpr int kDqCols = 16;

__device__ __forceinline__ float half_bits_to_float(uint16_t h) {
  _Float16 v;
  __builtin_memcpy(&v, &h, 2);
  return static_cast<float>(v);  // exact widening
}

// float -> bfloat16 bits, round to nearest even; NaN stays a quiet NaN
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// w_hat = fl(fl(alpha * level) + beta): the kernels are built without contraction
__device__ __forceinline__ float dequant_one(float alpha, float level, float beta) {
  const float prod = alpha * level;
  return prod + beta;
}

template <bool BF16_OUT, bool VEC>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const DequantDesc d) {
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
  if (VEC) {
    // K % 16 == 0, group % 16 == 0 and aligned pointers: 16 columns share one group
    for (int64_t c0 = int64_t(tid) * kDqCols; c0 < K; c0 += int64_t(kThreads) * kDqCols) {
      const uint2 cb = *reinterpret_cast<const uint2*>(codes + c0 / 2);
      const uint64_t nib = (uint64_t(cb.y) << 32) | cb.x;
      const int64_t g = c0 / d.group;
      const float alpha = half_bits_to_float(scale[g]);
      const float beta = half_bits_to_float(offset[g]);
      float w[kDqCols];
#pragma unroll
      for (int e = 0; e < kDqCols; ++e)
        w[e] = dequant_one(alpha, lut[(nib >> (4 * e)) & 0xF], beta);
      if (BF16_OUT) {
        uint32_t p[kDqCols / 2];
#pragma unroll
        for (int e = 0; e < kDqCols / 2; ++e)
          p[e] = bf16_rne_bits(w[2 * e]) | (bf16_rne_bits(w[2 * e + 1]) << 16);
        u32x4* dst = reinterpret_cast<u32x4*>(static_cast<uint16_t*>(d.out) + row * K + c0);
        __builtin_nontemporal_store(u32x4{p[0], p[1], p[2], p[3]}, dst);
        __builtin_nontemporal_store(u32x4{p[4], p[5], p[6], p[7]}, dst + 1);
      } else {
        f32x4* dst = reinterpret_cast<f32x4*>(static_cast<float*>(d.out) + row * K + c0);
#pragma unroll
        for (int v = 0; v < kDqCols / 4; ++v)
          __builtin_nontemporal_store(f32x4{w[4 * v], w[4 * v + 1], w[4 * v + 2], w[4 * v + 3]},
                                      dst + v);
      }
    }
  } else {
    for (int64_t j = tid; j < K; j += kThreads) {
      const uint8_t byte = codes[j / 2];
      const int q = (j & 1) ? (byte >> 4) : (byte & 0xF);
      const int64_t g = j / d.group;
      const float w = dequant_one(half_bits_to_float(scale[g]), lut[q], half_bits_to_float(offset[g]));
      if (BF16_OUT)
        static_cast<uint16_t*>(d.out)[row * K + j] = static_cast<uint16_t>(bf16_rne_bits(w));
      else
        static_cast<float*>(d.out)[row * K + j] = w;
    }
  }
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

}  // namespace

AbsmeanPlan plan_absmean(int64_t n_tokens, int64_t n_cols) {
  // about 1024 workgroups (4 per CU) and at least 64 tokens per slice
  const int64_t col_blocks = (n_cols + kAbsBlockChannels - 1) / kAbsBlockChannels;
  int64_t splits = (1024 + col_blocks - 1) / col_blocks;
  const int64_t max_splits = (n_tokens + 63) / 64;
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
  hipLaunchKernelGGL(absmean_finish_kernel, dim3(static_cast<uint32_t>((n_cols + kThreads - 1) / kThreads)),
                     dim3(kThreads), 0, stream, partial, plan.n_splits, n_tokens, n_cols, out);
  return hipGetLastError();
}

hipError_t launch_dequant(const DequantDesc& d, hipStream_t stream) {
  if (d.n_rows == 0) return hipSuccess;
  const bool vec = d.n_cols % kDqCols == 0 && d.group % kDqCols == 0 && aligned(d.codes, 8) &&
                   aligned(d.out, 16);
  const dim3 grid(static_cast<uint32_t>(d.n_rows));
  if (d.out_bf16 && vec)
    hipLaunchKernelGGL((dequant_kernel<true, true>), grid, dim3(kThreads), 0, stream, d);
  else if (d.out_bf16)
    hipLaunchKernelGGL((dequant_kernel<true, false>), grid, dim3(kThreads), 0, stream, d);
  else if (vec)
    hipLaunchKernelGGL((dequant_kernel<false, true>), grid, dim3(kThreads), 0, stream, d);
  else
    hipLaunchKernelGGL((dequant_kernel<false, false>), grid, dim3(kThreads), 0, stream, d);
  return hipGetLastError();
}

}  // namespace any4
