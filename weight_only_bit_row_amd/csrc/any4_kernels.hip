// gfx950 kernels of the any4 quantizer outside the row kernel: status clearing,
// emission from given assignments (stage entry point), the restart merge and the
// sorted-row Lloyd stage; and the host-side launch dispatch over row geometries.
// The row kernel itself is in any4_rows.h, instantiated by any4_rows_e*.hip.
#include "any4_rows.h"

#include <mutex>

namespace any4 {
namespace {

__global__ void clear_status_kernel(uint32_t* status) {
  if (threadIdx.x == 0) *status = 0u;
}

__global__ void copy_status_kernel(const uint32_t* src, uint32_t* dst) {
  if (threadIdx.x == 0) *dst = *src;
}

// Scratch of the entry point that allocates nothing (any4_quantize_noalloc): the status
// word and, with restarts, the candidate outputs.  Every device that runs the library
// holds its own copy until the process ends.  Host code must never pass `scratch` itself
// to a kernel (on the host it names a stand-in, not the device array): it uses the
// per-device address from noalloc_scratch() below.
static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

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

// Keep a restart's outputs for the rows where it beat the best objective so far.  One
// workgroup per row; every lane reads both objectives before lane 0 updates the best.
__global__ void restart_merge_kernel(MergeDesc d) {
  const int64_t row = blockIdx.x;
  const double cand = d.cand_obj[row];
  const bool take = cand < d.best_obj[row];  // NaN (a rejected row) is never taken
  __syncthreads();
  if (!take) return;
  const int64_t nb = d.n_cols / 2;
  for (int64_t i = threadIdx.x; i < nb; i += blockDim.x) d.codes[row * nb + i] = d.cand_codes[row * nb + i];
  if (threadIdx.x < d.n_clusters) {
    const int64_t j = row * d.n_clusters + threadIdx.x;
    d.lut[j] = d.cand_lut[j];
    if (d.c) d.c[j] = d.cand_c[j];
    if (d.picks) d.picks[j] = d.cand_picks[j];
  }
  if (threadIdx.x == 0) d.best_obj[row] = cand;
}

// ---------------------------------------------------------------------------------
// Sorted-row Lloyd (the Lloyd-Max form of Section 2.5's per-row 1-D clustering): the
// row's (w_S, a) pairs are sorted by w_S once and fp64 prefix sums P0 = sum a and
// P1 = sum a*w_S are taken in that order.  A round then needs, for the current
// centroids, the same exact fp32 switch points as the register path (so the same
// Eq. 18 assignment), one binary search per switch point, and two prefix differences
// per cluster for the Eq. 23 sums; the update itself is the register path's.  The
// sorted row and the prefix sums at the starts of its 256 chunks live in LDS:
//   [Smem][key: kp floats][a: kp floats][chunk bases: 2 x 257 fp64]
// with kp the row length rounded up to a power of two (padding keys +inf, a 0); a
// prefix sum inside a chunk is its base plus that chunk's elements added in order.
// ~40 KB at 4096 columns, so three rows share a CU; 133 KB at 16384, one row per CU.
constexpr int kSortedThreads = 256;
constexpr int kSortedRegs = 16;  // consecutive elements per thread in the register steps

// One bitonic step of stride STRIDE < kSortedRegs on a thread's kSortedRegs consecutive
// elements starting at index `base`: the same comparator as the LDS steps (ascending
// where bit `size` of the lower index is clear), so the network and its result are
// unchanged.
template <int STRIDE>
__device__ __forceinline__ void sort_step_regs(float (&kr)[kSortedRegs], float (&wr)[kSortedRegs], int base,
                                               int size) {
#pragma unroll
  for (int j = 0; j < kSortedRegs; ++j) {
    if ((j & STRIDE) == 0) {
      const bool up = ((base + j) & size) == 0;
      const float a = kr[j], b = kr[j + STRIDE];
      const bool sw = up ? (b < a) : (a < b);
      const float wa = wr[j], wb = wr[j + STRIDE];
      kr[j] = sw ? b : a;
      kr[j + STRIDE] = sw ? a : b;
      wr[j] = sw ? wb : wa;
      wr[j + STRIDE] = sw ? wa : wb;
    }
  }
}

// The steps of one `size` with strides 8, 4, 2, 1 (those below `size`), in registers.
__device__ __forceinline__ void sort_small_strides(float* key, float* wt, int tid, int size) {
  float kr[kSortedRegs], wr[kSortedRegs];
  const int base = tid * kSortedRegs;
#pragma unroll
  for (int v = 0; v < kSortedRegs / 4; ++v) {
    const float4 a = reinterpret_cast<const float4*>(key + base)[v];
    const float4 b = reinterpret_cast<const float4*>(wt + base)[v];
    kr[4 * v] = a.x; kr[4 * v + 1] = a.y; kr[4 * v + 2] = a.z; kr[4 * v + 3] = a.w;
    wr[4 * v] = b.x; wr[4 * v + 1] = b.y; wr[4 * v + 2] = b.z; wr[4 * v + 3] = b.w;
  }
  if (size > 8) sort_step_regs<8>(kr, wr, base, size);
  if (size > 4) sort_step_regs<4>(kr, wr, base, size);
  if (size > 2) sort_step_regs<2>(kr, wr, base, size);
  sort_step_regs<1>(kr, wr, base, size);
#pragma unroll
  for (int v = 0; v < kSortedRegs / 4; ++v) {
    reinterpret_cast<float4*>(key + base)[v] = make_float4(kr[4 * v], kr[4 * v + 1], kr[4 * v + 2], kr[4 * v + 3]);
    reinterpret_cast<float4*>(wt + base)[v] = make_float4(wr[4 * v], wr[4 * v + 1], wr[4 * v + 2], wr[4 * v + 3]);
  }
}

// Bitonic sort of kp (a power of two) (key, wt) pairs in LDS, ascending by key; each
// step pairs lo and lo + stride inside blocks of 2 * stride, the direction set by the
// bit `size` of lo.  A thread's pairs of a step (pair i = tid + 256 r) are all loaded
// before any is compared and stored, so their LDS reads are in flight together; every
// index belongs to one pair per step.  With kSortedRegs elements per thread
// (kp = 4096), the steps of stride below kSortedRegs stay inside a thread's consecutive
// elements and run in registers.  PER: compare pairs per thread, kp / 512 for the
// largest kp of the instance.  Ends with a block barrier.
template <int PER>
__device__ __forceinline__ void sort_pairs(float* key, float* wt, int kp, int tid) {
  const int half = kp / 2;
  const bool regs = kp == kSortedThreads * kSortedRegs;
  for (int size = 2; size <= kp; size <<= 1) {
    if (regs && size <= kSortedRegs) {
      if (size == kSortedRegs) {
        // sizes 2 .. 16 together: a thread's 16 elements hold whole blocks of each
        for (int sz = 2; sz <= kSortedRegs; sz <<= 1) {
          if (sz > 2) __syncthreads();
          sort_small_strides(key, wt, tid, sz);
        }
        __syncthreads();
      }
      continue;
    }
    const int last = regs ? kSortedRegs : 1;  // smallest stride taken in LDS
    for (int stride = size >> 1; stride >= last; stride >>= 1) {
      float k0[PER], k1[PER], w0[PER], w1[PER];
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int i = tid + r * kSortedThreads;
        if (i < half) {
          const int lo = 2 * i - (i & (stride - 1));
          k0[r] = key[lo];
          k1[r] = key[lo + stride];
          w0[r] = wt[lo];
          w1[r] = wt[lo + stride];
        }
      }
#pragma unroll
      for (int r = 0; r < PER; ++r) {
        const int i = tid + r * kSortedThreads;
        if (i < half) {
          const int lo = 2 * i - (i & (stride - 1));
          const bool up = (lo & size) == 0;
          if (up ? (k1[r] < k0[r]) : (k0[r] < k1[r])) {
            key[lo] = k1[r];
            key[lo + stride] = k0[r];
            wt[lo] = w1[r];
            wt[lo + stride] = w0[r];
          }
        }
      }
      __syncthreads();
    }
    if (regs) {
      sort_small_strides(key, wt, tid, size);
      __syncthreads();
    }
  }
}

// fp64 prefix sums of the first K sorted pairs at the starts of 256 chunks of
// C = ceil(K / 256) elements: thread t sums chunk t in order, thread 0 turns the chunk
// totals into chunk bases in thread order (tot[t] = P0 before chunk t, tot[TB + t] = P1,
// tot[256] and tot[TB + 256] the row's totals).  P(i) is then the base of chunk i / C
// plus the chunk's elements before i, added in order: one fixed order, so every sum is
// deterministic.  Ends with a block barrier.
constexpr int kSortedTB = kSortedThreads + 1;
__device__ __forceinline__ void chunk_bases(const float* key, const float* wt, int K, double* tot, int tid) {
  const int C = (K + kSortedThreads - 1) / kSortedThreads;
  {
    const int b0 = min(K, tid * C), b1 = min(K, b0 + C);
    double s0 = 0.0, s1 = 0.0;
    for (int i = b0; i < b1; ++i) {
      const double av = wt[i];
      s0 += av;
      s1 += av * static_cast<double>(key[i]);
    }
    tot[tid] = s0;
    tot[kSortedTB + tid] = s1;
  }
  __syncthreads();
  if (tid == 0) {
    double r0 = 0.0, r1 = 0.0;
    for (int t = 0; t < kSortedThreads; ++t) {
      const double v0 = tot[t], v1 = tot[kSortedTB + t];
      tot[t] = r0;
      tot[kSortedTB + t] = r1;
      r0 += v0;
      r1 += v1;
    }
    tot[kSortedThreads] = r0;
    tot[kSortedTB + kSortedThreads] = r1;
  }
  __syncthreads();
}

// Number of the first n keys below th (keys ascending).
__device__ __forceinline__ int keys_below(const float* key, int n, float th) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (key[mid] < th)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo;
}

// Per lane p < U of wave 0: the Eq. 23 sums of sorted position p from the prefix sums
// (q0, q1) at its right end; writes them to S.wred[0] for update_and_structure.
__device__ __forceinline__ void publish_position_sums(Smem& S, int lane, int U, double q0, double q1) {
  const double p0 = __shfl_up(q0, 1), p1 = __shfl_up(q1, 1);
  if (lane < kMaxClusters) {
    double c0 = 0.0, c1 = 0.0;
    if (lane < U) {
      c0 = (lane == 0) ? q0 : q0 - p0;
      c1 = (lane == 0) ? q1 : q1 - p1;
      if (!(c0 > 0.0)) c0 = c1 = 0.0;  // an empty range (or an unordered pair) adds nothing
    }
    S.wred[0][lane] = c0;
    S.wred[0][kMaxClusters + lane] = c1;
  }
  wave_lds_fence();
}

template <int PER>
__global__ __launch_bounds__(kSortedThreads) void sorted_lloyd_kernel(const SortedDesc d) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  const int K = d.n_cols, kp = d.kp, k = d.n_clusters, tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  float* key = reinterpret_cast<float*>(smem_raw + kSmemHdr);
  float* wt = key + kp;
  double* tot = reinterpret_cast<double*>(wt + kp);  // [2][kSortedThreads + 1]
  constexpr int TB = kSortedTB;
  const int64_t row = blockIdx.x;
  const float* ws = d.w_s + row * K;
  const float* ar = d.a + row * K;
  for (int i = tid; i < kp; i += kSortedThreads) {
    key[i] = i < K ? ws[i] : __builtin_huge_valf();
    wt[i] = i < K ? ar[i] : 0.0f;
  }
  if (tid < k) S.c[tid] = d.c_in[row * k + tid];
  __syncthreads();
  sort_pairs<PER>(key, wt, kp, tid);
  chunk_bases(key, wt, K, tot, tid);
  const int C = (K + kSortedThreads - 1) / kSortedThreads;
  // the rounds run on wave 0 alone (no block barrier from here on)
  if (tid >= kWave) return;
  const float off = d.symmetric ? static_cast<float>(k / 2) : 0.0f;
  const int G = kCellsPerUnit * k;
  float sv, t;
  int si;
  uint32_t tc;
  int U = build_structure(S, k, G, off, lane, t, tc, sv, si);
  for (int it = 0; it < d.iters; ++it) {
    // lane p < U - 1: the number of keys below switch point p (elements at or above it
    // sit right of sorted position p, the register path's rule)
    const int idx = (lane + 1 < U) ? keys_below(key, K, S.thr[lane]) : K;
    // prefix sums at the switch index (lane p < U - 1) or at K (the last position)
    double q0 = 0.0, q1 = 0.0;
    if (lane < U) {
      const int ch = min(idx / C, kSortedThreads);
      q0 = tot[ch];
      q1 = tot[TB + ch];
      for (int i = ch * C; i < idx; ++i) {
        const double av = wt[i];
        q0 += av;
        q1 += av * static_cast<double>(key[i]);
      }
    }
    publish_position_sums(S, lane, U, q0, q1);
    bool same;
    U = update_and_structure(S, 1, k, G, off, lane, U, sv, si, t, tc, same);
  }
  if (lane < k) d.c_out[row * k + lane] = S.c[lane];
}

// Rows of kSortedMaxCols + 2 .. 2 kSortedMaxCols columns: the row is sorted as two
// halves, A = columns [0, K/2) and B = [K/2, K), each padded to kSortedMaxCols and
// sorted in LDS in turn with its own chunk bases.  The sorted sample weights of both
// halves go to the caller's workspace (B's keys pass through it while A is sorted), and
// the rounds keep both halves' keys and chunk bases in LDS:
//   [Smem][keys A: kh floats][keys B: kh floats][chunk bases A, B: 2 x 2 x 257 fp64]
// A cluster's Eq. 23 sums are the sums over the two halves: each switch point is
// searched in both, and a prefix sum is P_A + P_B at the two indices, the in-chunk
// weights read from the workspace.  Workspace per row: keys B, weights A, weights B,
// kh floats each.
constexpr int kSortedChunkMax = kSortedMaxCols / kSortedThreads;  // chunk length bound
__device__ __forceinline__ void half_prefix(const float* key, const float* wt_g, const double* tot, int n, int at,
                                            double& q0, double& q1) {
  // chunk base at `at`, then the chunk's elements before `at` in order; the weights come
  // from global memory, all loads issued first (indices clamped into the half)
  const int C = (n + kSortedThreads - 1) / kSortedThreads;
  const int ch = min(at / C, kSortedThreads);
  const int base = ch * C;
  q0 = tot[ch];
  q1 = tot[kSortedTB + ch];
  float wv[kSortedChunkMax];
#pragma unroll
  for (int j = 0; j < kSortedChunkMax; ++j) wv[j] = wt_g[min(base + j, n - 1)];
#pragma unroll
  for (int j = 0; j < kSortedChunkMax; ++j) {
    if (base + j < at) {
      const double av = wv[j];
      q0 += av;
      q1 += av * static_cast<double>(key[base + j]);
    }
  }
}

__global__ __launch_bounds__(kSortedThreads) void sorted_lloyd_split_kernel(const SortedDesc d) {
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
  Smem& S = *reinterpret_cast<Smem*>(smem_raw);
  constexpr int kh = kSortedMaxCols;
  const int K = d.n_cols, KA = K / 2, KB = K - KA, k = d.n_clusters, tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  float* key = reinterpret_cast<float*>(smem_raw + kSmemHdr);  // [2 kh]
  double* totA = reinterpret_cast<double*>(key + 2 * kh);      // [2][257]
  double* totB = totA + 2 * kSortedTB;
  const int64_t row = blockIdx.x;
  const float* ws = d.w_s + row * K;
  const float* ar = d.a + row * K;
  float* keyB_g = d.work + row * (3 * static_cast<int64_t>(kh));
  float* wtA_g = keyB_g + kh;
  float* wtB_g = wtA_g + kh;
  if (tid < k) S.c[tid] = d.c_in[row * k + tid];
  // half B: sort in the whole key area (keys, then weights), bases, out to the workspace
  for (int i = tid; i < kh; i += kSortedThreads) {
    key[i] = i < KB ? ws[KA + i] : __builtin_huge_valf();
    key[kh + i] = i < KB ? ar[KA + i] : 0.0f;
  }
  __syncthreads();
  sort_pairs<kSortedMaxCols / 2 / kSortedThreads>(key, key + kh, kh, tid);
  chunk_bases(key, key + kh, KB, totB, tid);
  for (int i = tid; i < KB; i += kSortedThreads) {
    keyB_g[i] = key[i];
    wtB_g[i] = key[kh + i];
  }
  __syncthreads();
  // half A: the same, its keys stay in the first half of the area
  for (int i = tid; i < kh; i += kSortedThreads) {
    key[i] = i < KA ? ws[i] : __builtin_huge_valf();
    key[kh + i] = i < KA ? ar[i] : 0.0f;
  }
  __syncthreads();
  sort_pairs<kSortedMaxCols / 2 / kSortedThreads>(key, key + kh, kh, tid);
  chunk_bases(key, key + kh, KA, totA, tid);
  for (int i = tid; i < KA; i += kSortedThreads) wtA_g[i] = key[kh + i];
  __syncthreads();  // every weight of A is read before B's keys replace them
  for (int i = tid; i < KB; i += kSortedThreads) key[kh + i] = keyB_g[i];
  __syncthreads();  // also orders this workgroup's workspace stores before the rounds' loads
  const float* keyA = key;
  const float* keyB = key + kh;
  // the rounds run on wave 0 alone (no block barrier from here on)
  if (tid >= kWave) return;
  const float off = d.symmetric ? static_cast<float>(k / 2) : 0.0f;
  const int G = kCellsPerUnit * k;
  float sv, t;
  int si;
  uint32_t tc;
  int U = build_structure(S, k, G, off, lane, t, tc, sv, si);
  for (int it = 0; it < d.iters; ++it) {
    int ia = KA, ib = KB;
    if (lane + 1 < U) {
      const float th = S.thr[lane];
      ia = keys_below(keyA, KA, th);
      ib = keys_below(keyB, KB, th);
    }
    double q0 = 0.0, q1 = 0.0;
    if (lane < U) {
      double a0, a1, b0, b1;
      half_prefix(keyA, wtA_g, totA, KA, ia, a0, a1);
      half_prefix(keyB, wtB_g, totB, KB, ib, b0, b1);
      q0 = a0 + b0;
      q1 = a1 + b1;
    }
    publish_position_sums(S, lane, U, q0, q1);
    bool same;
    U = update_and_structure(S, 1, k, G, off, lane, U, sv, si, t, tc, same);
  }
  if (lane < k) d.c_out[row * k + lane] = S.c[lane];
}

}  // namespace

hipError_t launch_rows(const LaunchArgs& args, RowConfig cfg, int mode, int64_t n_blocks,
                       hipStream_t stream) {
  if (n_blocks <= 0) return hipSuccess;
  // choose_config gives 8 or 16 elements per lane only on one wave, 32 on 1-16 waves.
  // Rows of 5 or more waves take the 1024-lane instance: at 128 VGPRs (sampling weights
  // in the bin area) two rows of 5-8 waves share a CU, 18-27% faster than one row at
  // 168 VGPRs.  Rows of 2-4 waves take it too on the default path (eight 2-wave rows per
  // CU instead of six, now that the rounds no longer saturate the LDS: 1.5-3% faster);
  // with a method variant they keep the 2-4-wave instance, tuned for the variants'
  // narrow-group scaling.
  if (cfg.nw == 1) {
    switch (cfg.e) {
      case 8: return launch_rows_e8(args, mode, n_blocks, stream);
      case 16: return launch_rows_e16(args, mode, n_blocks, stream);
      case 32: return launch_rows_e32_w1(args, mode, n_blocks, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (cfg.e != 32 || cfg.nw > 16) return hipErrorInvalidValue;
  const bool var = args.variant != 0 || args.restart != 0;
  return (cfg.nw > 4 || !var) ? launch_rows_e32_w16(args, mode, n_blocks, stream)
                              : launch_rows_e32_w8(args, mode, n_blocks, stream);
}

hipError_t launch_restart_merge(const MergeDesc& d, hipStream_t stream) {
  if (d.n_rows == 0) return hipSuccess;
  hipLaunchKernelGGL(restart_merge_kernel, dim3(static_cast<unsigned>(d.n_rows)), dim3(256), 0,
                     stream, d);
  return hipGetLastError();
}

size_t sorted_lloyd_lds_bytes(int64_t n_cols) {
  if (n_cols > kSortedMaxCols)  // two halves: both halves' keys and chunk bases
    return kSmemHdr + 2 * sizeof(float) * static_cast<size_t>(kSortedMaxCols) +
           4 * sizeof(double) * (kSortedThreads + 1);
  int64_t kp = 2;
  while (kp < n_cols) kp <<= 1;
  return kSmemHdr + 2 * sizeof(float) * static_cast<size_t>(kp) + 2 * sizeof(double) * (kSortedThreads + 1);
}

size_t sorted_lloyd_work_bytes(int64_t n_rows, int64_t n_cols) {
  return n_cols > kSortedMaxCols ? static_cast<size_t>(n_rows) * 3 * sizeof(float) * kSortedMaxCols : 0;
}

hipError_t launch_sorted_lloyd(SortedDesc d, hipStream_t stream) {
  if (d.n_rows == 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(d.n_rows));
  if (d.n_cols > kSortedMaxCols) {
    d.kp = kSortedMaxCols;
    hipLaunchKernelGGL(sorted_lloyd_split_kernel, grid, dim3(kSortedThreads), sorted_lloyd_lds_bytes(d.n_cols),
                       stream, d);
    return hipGetLastError();
  }
  int kp = 2;
  while (kp < d.n_cols) kp <<= 1;
  d.kp = kp;
  // rows up to 4096 columns take the instance with 8 pairs per thread (its step registers
  // sized for them); longer rows up to kSortedMaxCols the one with 32
  constexpr int kSmallCols = kSortedThreads * kSortedRegs;
  static_assert(kSortedMaxCols == 4 * kSmallCols, "the large instance covers 4x the small one");
  if (kp <= kSmallCols)
    hipLaunchKernelGGL((sorted_lloyd_kernel<kSmallCols / 2 / kSortedThreads>), grid, dim3(kSortedThreads),
                       sorted_lloyd_lds_bytes(d.n_cols), stream, d);
  else
    hipLaunchKernelGGL((sorted_lloyd_kernel<kSortedMaxCols / 2 / kSortedThreads>), grid, dim3(kSortedThreads),
                       sorted_lloyd_lds_bytes(d.n_cols), stream, d);
  return hipGetLastError();
}

// Device address of `scratch` on the current device, looked up once per device (under a
// lock, so concurrent first calls are safe) and kept.
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_lock;
unsigned char* g_scratch[kMaxScratchDevices];

hipError_t noalloc_scratch(unsigned char** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> guard(g_scratch_lock);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<unsigned char*>(ptr);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

hipError_t launch_copy_status(const uint32_t* src, uint32_t* dst, hipStream_t stream) {
  hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(64), 0, stream, src, dst);
  return hipGetLastError();
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
