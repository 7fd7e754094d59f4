// Column absolute maxima and smoothing factors (gfx950).
//
// Column absmax (inferenceinterviews.com "Why do activation outliers break INT8
// W8A8...", section "A strong answer": max over tokens t of |X_tj| and over
// output rows n of |W_nj|) is a pure HBM stream: each element is read once.
// Two forms: a slab form (bf16) in which a workgroup's 64 lanes each own one
// 16-byte column chunk and its 4 waves walk interleaved rows of a short row
// slab, so every wave load is 1 KB of one row, the 4 partial maxima meeting in
// LDS; and a column-block form (fp32) described at its kernel.  Either way one
// atomic max per column and slab goes to the output: |x| >= 0, so the unsigned
// order of the binary32 bit patterns is the numeric order and an integer atomic
// max is exact.  The per-tensor range of the smoothed activations and the
// smoothing factors are here too.
#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace sq {

__global__ void fill_f32_kernel(float* __restrict__ p, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void fill2_f32_kernel(float* __restrict__ p, float* __restrict__ q, int64_t n, float v) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    p[i] = v;
    q[i] = v;
  }
}

// Element loaders: VEC elements of one row starting at column c.
template <typename T, int VEC> struct ChunkLoad;
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
// 16 bytes, with a non-temporal hint when NT (data read once: it then does not
// displace what a following kernel reads again from the Infinity Cache).
template <bool NT> __device__ __forceinline__ f32x4_t load16f(const float* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  else return *reinterpret_cast<const f32x4_t*>(p);
}
template <bool NT> __device__ __forceinline__ u32x4_t load16u(const uint16_t* p) {
  if constexpr (NT) return __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  else return *reinterpret_cast<const u32x4_t*>(p);
}

template <> struct ChunkLoad<float, 4> {
  template <bool NT = false> static __device__ __forceinline__ void abs(const float* p, float* o) {
    const f32x4_t v = load16f<NT>(p);
    o[0] = fabsf(v[0]); o[1] = fabsf(v[1]); o[2] = fabsf(v[2]); o[3] = fabsf(v[3]);
  }
};
template <> struct ChunkLoad<uint16_t, 8> {
  template <bool NT = false> static __device__ __forceinline__ void abs(const uint16_t* p, float* o) {
    uint4 v = *reinterpret_cast<const uint4*>(p);
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = fabsf(bf16_lo(w[i]));
      o[2 * i + 1] = fabsf(bf16_hi(w[i]));
    }
  }
};
template <> struct ChunkLoad<float, 1> {
  template <bool NT = false> static __device__ __forceinline__ void abs(const float* p, float* o) { o[0] = fabsf(*p); }
};
template <> struct ChunkLoad<uint16_t, 1> {
  template <bool NT = false> static __device__ __forceinline__ void abs(const uint16_t* p, float* o) {
    o[0] = fabsf(bf16_to_f32(*p));
  }
};

// Running maximum of |x| over a chunk of VEC columns.  bf16 chunks keep four
// packed pairs of 16-bit patterns with the sign bits cleared: for non-negative
// bf16 values the unsigned order of the patterns is the numeric order, so one
// packed unsigned max handles two columns.
typedef unsigned short us2 __attribute__((ext_vector_type(2)));

template <typename T, int VEC> struct ColMax {
  float m[VEC];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int i = 0; i < VEC; ++i) m[i] = 0.0f;
  }
  template <bool NT = false> __device__ __forceinline__ void add(const T* p) {
    float a[VEC];
    ChunkLoad<T, VEC>::template abs<NT>(p, a);
#pragma unroll
    for (int i = 0; i < VEC; ++i) m[i] = fmaxf(m[i], a[i]);
  }
  __device__ __forceinline__ void result(float* o) const {
#pragma unroll
    for (int i = 0; i < VEC; ++i) o[i] = m[i];
  }
};
template <> struct ColMax<uint16_t, 8> {
  uint32_t pm[4];
  __device__ __forceinline__ void init() { pm[0] = pm[1] = pm[2] = pm[3] = 0u; }
  template <bool NT = false> __device__ __forceinline__ void add(const uint16_t* p) {
    const u32x4_t v = load16u<NT>(p);
    const uint32_t w[4] = {v[0] & 0x7FFF7FFFu, v[1] & 0x7FFF7FFFu, v[2] & 0x7FFF7FFFu, v[3] & 0x7FFF7FFFu};
#pragma unroll
    for (int q = 0; q < 4; ++q)
      pm[q] = __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(us2, pm[q]),
                                                                     __builtin_bit_cast(us2, w[q])));
  }
  __device__ __forceinline__ void result(float* o) const {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      o[2 * q] = __uint_as_float(pm[q] << 16);
      o[2 * q + 1] = __uint_as_float(pm[q] & 0xFFFF0000u);
    }
  }
};

// grid.x: groups of 64 chunks; grid.y: row slabs of `slab` rows.  Each wave
// keeps U rows (of its 1 KB column strip) in flight.
template <typename T, int VEC, int U>
__global__ __launch_bounds__(256) void col_absmax_kernel(const T* __restrict__ A, int64_t rows,
                                                         int64_t cols, int64_t slab,
                                                         float* __restrict__ amax) {
  __shared__ float part[4][64][VEC];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * VEC;
  const bool active = c0 < cols;   // cols % VEC == 0 on this path
  const int64_t r_begin = (int64_t)blockIdx.y * slab;
  const int64_t r_end = r_begin + slab < rows ? r_begin + slab : rows;
  ColMax<T, VEC> acc;
  acc.init();
  if (active) {
    const T* p = A + c0;
    int64_t r = r_begin + wave;
    for (; r + 4 * (U - 1) < r_end; r += 4 * U) {
#pragma unroll
      for (int u = 0; u < U; ++u) acc.add(p + (r + 4 * u) * cols);
    }
    for (; r < r_end; r += 4) acc.add(p + r * cols);
  }
  float m[VEC];
  acc.result(m);
#pragma unroll
  for (int i = 0; i < VEC; ++i) part[wave][lane][i] = m[i];
  __syncthreads();
  if (wave == 0 && active) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) {
      float v = fmaxf(fmaxf(part[0][lane][i], part[1][lane][i]),
                      fmaxf(part[2][lane][i], part[3][lane][i]));
      atomicMax(reinterpret_cast<unsigned int*>(amax + c0 + i), __float_as_uint(v));
    }
  }
}

// Column-block form: the 256 threads of a workgroup sit side by side over a
// block of 256 16-byte column chunks (4 KB of each row) and walk every S-th row
// starting at row y, U rows of loads in flight, then issue one atomic max per
// column.  Interleaved rows keep the rows read at any moment by all workgroups
// one contiguous region of the matrix (8192 x 8192 fp32: 43 us, against 47 us for
// contiguous row slabs and 55 us for the slab form, whose 4 waves split the rows
// of short slabs; for bf16 alone the slab form stays ahead).  Rows past the end
// repeat the workgroup's previous row (harmless for a maximum), so the loads
// carry no conditions.  Requires S <= rows and 16-byte aligned rows.
template <typename T, int U, bool NT = false>
__device__ __forceinline__ void colmax_block(const T* __restrict__ A, int64_t rows, int64_t cols, int64_t x,
                                             int64_t y, int64_t S, float* __restrict__ amax) {
  constexpr int VEC = 16 / sizeof(T);
  const int64_t c0 = (x * 256 + threadIdx.x) * VEC;
  if (c0 >= cols) return;   // cols % VEC == 0 on this path
  ColMax<T, VEC> acc;
  acc.init();
  const T* p = A + c0;
  int64_t last = y;
  for (int64_t r = y; r < rows; r += S * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t rr = r + u * S;
      acc.template add<NT>(p + (rr < rows ? rr : last) * cols);
    }
    last = r;
  }
  float m[VEC];
  acc.result(m);
#pragma unroll
  for (int i = 0; i < VEC; ++i) atomicMax(reinterpret_cast<unsigned int*>(amax + c0 + i), __float_as_uint(m[i]));
}

// grid (column blocks, S)
template <typename T, int U>
__global__ __launch_bounds__(256) void col_absmax_blk_kernel(const T* __restrict__ A, int64_t rows,
                                                             int64_t cols, float* __restrict__ amax) {
  colmax_block<T, U>(A, rows, cols, blockIdx.x, blockIdx.y, gridDim.y, amax);
}

// Both column maxima of the smoothing factors in one launch: workgroups
// [0, cbX*SX) take the column blocks of X (rows y, y + SX, ...), the others those
// of W.  SX and SW are chosen so that every workgroup reads about the same
// bytes, about one workgroup per CU in all; the two streams then share the chip
// instead of following each other (8192 x 8192 bf16 X and fp32 W: 66 us against
// 78 us for the two launches).  X is read with non-temporal loads: the calibration
// activations are not read again, while W is quantised next, and with X out of
// the Infinity Cache more of W is still there (pass and weight quantiser together
// ~6 us faster on 8192 x 8192; W read that way too made the quantiser 16 us
// slower).
template <typename TX, typename TW, int U>
__global__ __launch_bounds__(256) void col_absmax_pair_kernel(const TX* __restrict__ X, int64_t T, int64_t cbX,
                                                              int64_t SX, const TW* __restrict__ W, int64_t N,
                                                              int64_t cbW, int64_t SW, int64_t K,
                                                              float* __restrict__ xa, float* __restrict__ wa) {
  const int64_t g = blockIdx.x, nX = cbX * SX;
  if (g < nX) {
    colmax_block<TX, U, true>(X, T, K, g % cbX, g / cbX, SX, xa);
  } else {
    const int64_t h = g - nX;
    colmax_block<TW, U>(W, N, K, h % cbW, h / cbW, SW, wa);
  }
}

// Range of the whole smoothed activation tensor, max over t, k of
// |fl32(A_tk / s_k)| (the per-tensor activation levels of multigrid.ai
// "SmoothQuant Explained", section "Where it fits, and where it does not").
// Rounded division by |s_k| is monotone in |A_tk|, and rounding to nearest is
// symmetric, so each column's largest quotient is fl32(max_t |A_tk| / |s_k|):
// the workgroup takes the column maxima of |A| over its row slab exactly as
// col_absmax_kernel does, divides once per column, reduces to one value and
// issues a single atomic max (instead of one per column).
template <typename T, int VEC, int U, bool HAS_S>
__global__ __launch_bounds__(256) void tensor_absmax_kernel(const T* __restrict__ A, int64_t rows,
                                                            int64_t cols, int64_t slab,
                                                            const float* __restrict__ s,
                                                            float* __restrict__ amax) {
  __shared__ float part[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t c0 = ((int64_t)blockIdx.x * 64 + lane) * VEC;
  const bool active = c0 < cols;   // cols % VEC == 0 on this path
  const int64_t r_begin = (int64_t)blockIdx.y * slab;
  const int64_t r_end = r_begin + slab < rows ? r_begin + slab : rows;
  ColMax<T, VEC> acc;
  acc.init();
  if (active) {
    const T* p = A + c0;
    int64_t r = r_begin + wave;
    for (; r + 4 * (U - 1) < r_end; r += 4 * U) {
#pragma unroll
      for (int u = 0; u < U; ++u) acc.add(p + (r + 4 * u) * cols);
    }
    for (; r < r_end; r += 4) acc.add(p + r * cols);
  }
  float m[VEC];
  acc.result(m);
  float v = 0.0f;
  if (active) {
#pragma unroll
    for (int i = 0; i < VEC; ++i) v = fmaxf(v, HAS_S ? m[i] / fabsf(s[c0 + i]) : m[i]);
  }
  v = wave_max_nonneg(v);
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (threadIdx.x == 0)
    atomicMax(reinterpret_cast<unsigned int*>(amax),
              __float_as_uint(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]))));
}

// Same range, row-walking form for rows of at most 16384 elements that are
// 16-byte aligned multiples of 8: a workgroup owns whole rows (thread t holds
// the 8-element chunks t, t + 256, ...), walks row groups r0 = U * blockIdx.x,
// + U * gridDim.x, ... and issues the loads of U complete rows before folding
// them into per-column running maxima of |A| (packed for bf16).  Every HBM read
// is a contiguous row; the last group reuses row R-1 in place of rows past the
// end (harmless for a maximum) and chunks past the row end re-read its last
// chunk, so the loads carry no conditions.
template <typename T, bool HAS_S, int CPT, int U, bool FULL>
__global__ __launch_bounds__(256) void tensor_absmax_rows_kernel(const T* __restrict__ A, int64_t R,
                                                                 int64_t K,
                                                                 const float* __restrict__ s,
                                                                 float* __restrict__ amax) {
  __shared__ float part[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nchunks = K >> 3;
  constexpr int VEC = 16 / sizeof(T) < 8 ? 16 / sizeof(T) : 8;   // elements per 16-byte load
  constexpr int LPC = 8 / VEC;                                     // loads per 8-element chunk
  ColMax<T, VEC> acc[CPT][LPC];
#pragma unroll
  for (int j = 0; j < CPT; ++j)
#pragma unroll
    for (int h = 0; h < LPC; ++h) acc[j][h].init();
  for (int64_t r0 = (int64_t)blockIdx.x * U; r0 < R; r0 += (int64_t)gridDim.x * U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = r0 + u < R ? r0 + u : R - 1;
#pragma unroll
      for (int j = 0; j < CPT; ++j) {
        // chunks past the row end re-read the last chunk; their maxima are
        // ignored below
        int64_t c = (int64_t)j * 256 + tid;
        if (!FULL && c >= nchunks) c = nchunks - 1;
#pragma unroll
        for (int h = 0; h < LPC; ++h) acc[j][h].add(A + r * K + c * 8 + h * VEC);
      }
    }
  }
  float v = 0.0f;
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = (int64_t)j * 256 + tid;
    if (FULL || c < nchunks) {
#pragma unroll
      for (int h = 0; h < LPC; ++h) {
        float m[VEC];
        acc[j][h].result(m);
#pragma unroll
        for (int i = 0; i < VEC; ++i)
          v = fmaxf(v, HAS_S ? m[i] / fabsf(s[c * 8 + h * VEC + i]) : m[i]);
      }
    }
  }
  v = wave_max_nonneg(v);
  if (lane == 0) part[wave] = v;
  __syncthreads();
  if (tid == 0)
    atomicMax(reinterpret_cast<unsigned int*>(amax),
              __float_as_uint(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]))));
}

// s_j = max(xa_j, 1e-8)^alpha / max(wa_j, 1e-8)^(1 - alpha), binary64, rounded once
// (multigrid.ai "SmoothQuant Explained", section "Alpha: how much difficulty to
// move"; 1e-8 floor from the maitreyasuin page, section "Route it, or move it").
__device__ __forceinline__ float smooth_factor(float xa, float wa, double alpha) {
  const float eps = 1e-8f;
  const float x = xa < eps ? eps : xa;
  const float w = wa < eps ? eps : wa;
  double r;
  if (alpha == 0.0) {
    r = 1.0 / (double)w;                 // the alpha = 0 form, exactly
  } else if (alpha == 1.0) {
    r = (double)x;                       // the alpha = 1 form, exactly
  } else {
    r = pow((double)x, alpha) / pow((double)w, 1.0 - alpha);
  }
  return (float)r;
}

// xa may alias s (each entry is read, then written, by one thread).
__global__ void smooth_scales_kernel(const float* xa, const float* __restrict__ wa, int64_t K, double alpha,
                                     float* s) {
  int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  s[j] = smooth_factor(xa[j], wa[j], alpha);
}

// Smoothing factors whose weight maxima are formed inside one workgroup, for
// callers that keep no [K] buffer of weight maxima: a workgroup owns a strip of
// columns over all N rows of W, so each column's maximum is final when its
// waves meet in LDS, and the workgroup then writes s_j = factor(xa_j, wa_j) for
// its columns.  Vector form (16-byte aligned rows): a strip is 128 bytes of each
// row (32 fp32 / 64 bf16 columns); lane l reads 16-byte chunk l % 8 of row
// l / 8 of an 8-row group, the 4 waves take successive 8-row groups, U groups of
// loads in flight.  xa may alias s: each column is read, then written, by the
// same thread, after every load of W.
template <typename T, int U>
__global__ __launch_bounds__(256) void smooth_wstrip_kernel(const T* __restrict__ W, int64_t N, int64_t K,
                                                            const float* xa, double alpha, float* s) {
  constexpr int VEC = 16 / sizeof(T);
  constexpr int SC = 8 * VEC;   // columns per strip
  __shared__ float part[32][SC];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int chunk = lane & 7, rsub = lane >> 3;
  const int64_t c0 = (int64_t)blockIdx.x * SC + chunk * VEC;
  ColMax<T, VEC> acc;
  acc.init();
  if (c0 < K) {   // K % VEC == 0 on this path
    const T* p = W + c0;
    int64_t r = (int64_t)wave * 8 + rsub;
    for (; r + 32 * (U - 1) < N; r += 32 * U) {
#pragma unroll
      for (int u = 0; u < U; ++u) acc.add(p + (r + 32 * u) * K);
    }
    for (; r < N; r += 32) acc.add(p + r * K);
  }
  float m[VEC];
  acc.result(m);
#pragma unroll
  for (int i = 0; i < VEC; ++i) part[wave * 8 + rsub][chunk * VEC + i] = m[i];
  __syncthreads();
  if (tid < SC) {
    const int64_t j = (int64_t)blockIdx.x * SC + tid;
    if (j < K) {
      float w = 0.0f;
#pragma unroll
      for (int g = 0; g < 32; ++g) w = fmaxf(w, part[g][tid]);
      s[j] = smooth_factor(xa[j], w, alpha);
    }
  }
}

// Scalar form of the same (any alignment): lane l owns column 64 * blockIdx.x + l,
// the 4 waves take rows wave, wave + 4, ...
template <typename T, int U>
__global__ __launch_bounds__(256) void smooth_wcol_kernel(const T* __restrict__ W, int64_t N, int64_t K,
                                                          const float* xa, double alpha, float* s) {
  __shared__ float part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * 64 + lane;
  ColMax<T, 1> acc;
  acc.init();
  if (j < K) {
    const T* p = W + j;
    int64_t r = wave;
    for (; r + 4 * (U - 1) < N; r += 4 * U) {
#pragma unroll
      for (int u = 0; u < U; ++u) acc.add(p + (r + 4 * u) * K);
    }
    for (; r < N; r += 4) acc.add(p + r * K);
  }
  float m;
  acc.result(&m);
  part[wave][lane] = m;
  __syncthreads();
  if (wave == 0 && j < K)
    s[j] = smooth_factor(xa[j], fmaxf(fmaxf(part[0][lane], part[1][lane]), fmaxf(part[2][lane], part[3][lane])),
                         alpha);
}

static int grid_1d(int64_t n, int threads, int cap) {
  int64_t g = (n + threads - 1) / threads;
  return (int)(g < cap ? (g < 1 ? 1 : g) : cap);
}

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st) {
  SQ_TRACE("fill %lld floats with %g", (long long)n, (double)v);
  hipLaunchKernelGGL(fill_f32_kernel, dim3(grid_1d(n, 256, 1024)), dim3(256), 0, st, p, n, v);
  return hipGetLastError();
}

hipError_t launch_fill2(float* p, float* q, int64_t n, float v, hipStream_t st) {
  SQ_TRACE("fill 2 x %lld floats with %g", (long long)n, (double)v);
  hipLaunchKernelGGL(fill2_f32_kernel, dim3(grid_1d(n, 256, 1024)), dim3(256), 0, st, p, q, n, v);
  return hipGetLastError();
}

template <typename T, int VEC, int U>
static hipError_t col_absmax_t(const T* A, int64_t rows, int64_t cols, float* amax, int ncu,
                               hipStream_t st) {
  const int64_t chunks = (cols + VEC - 1) / VEC;
  const int64_t gx = (chunks + 63) / 64;
  const int64_t target = 8LL * ncu;                 // workgroups to fill the chip
  int64_t slabs = target / gx;
  if (slabs < 1) slabs = 1;
  int64_t max_slabs = (rows + 15) / 16;             // at least 16 rows per slab
  if (slabs > max_slabs) slabs = max_slabs;
  if (slabs > 65535) slabs = 65535;
  int64_t slab = (rows + slabs - 1) / slabs;
  slabs = (rows + slab - 1) / slab;
  SQ_TRACE("col_absmax (%s, %d elements per load, %d rows in flight) rows %lld cols %lld, grid %lld x %lld slabs of %lld rows",
           sizeof(T) == 2 ? "bf16" : "f32", VEC, U, (long long)rows, (long long)cols, (long long)gx, (long long)slabs,
           (long long)slab);
  hipLaunchKernelGGL((col_absmax_kernel<T, VEC, U>), dim3((unsigned)gx, (unsigned)slabs), dim3(256), 0,
                     st, A, rows, cols, slab, amax);
  return hipGetLastError();
}

template <typename TX, typename TW>
static hipError_t col_absmax_pair_t(const void* X, int64_t T, const void* W, int64_t N, int64_t K, float* xa,
                                    float* wa, int ncu, hipStream_t st) {
  const double bx = (double)T * K * sizeof(TX), bw = (double)N * K * sizeof(TW);
  const int64_t cbX = (K * (int64_t)sizeof(TX) + 4095) / 4096, cbW = (K * (int64_t)sizeof(TW) + 4095) / 4096;
  auto interleave = [&](double share, int64_t cb, int64_t rows) {
    int64_t S = (int64_t)(ncu * share / cb + 0.5);
    if (S < 1) S = 1;
    if (S > rows) S = rows;
    return S;
  };
  const int64_t SX = interleave(bx / (bx + bw), cbX, T), SW = interleave(bw / (bx + bw), cbW, N);
  SQ_TRACE("col_absmax_pair (X %s T %lld: %lld column blocks x %lld row interleave; W %s N %lld: %lld x %lld) K %lld, "
           "grid %lld x 256 threads",
           sizeof(TX) == 2 ? "bf16" : "f32", (long long)T, (long long)cbX, (long long)SX, sizeof(TW) == 2 ? "bf16" : "f32",
           (long long)N, (long long)cbW, (long long)SW, (long long)K, (long long)(cbX * SX + cbW * SW));
  hipLaunchKernelGGL((col_absmax_pair_kernel<TX, TW, 8>), dim3((unsigned)(cbX * SX + cbW * SW)), dim3(256), 0, st,
                     static_cast<const TX*>(X), T, cbX, SX, static_cast<const TW*>(W), N, cbW, SW, K, xa, wa);
  return hipGetLastError();
}

hipError_t launch_col_absmax_pair(const void* X, bool x_bf16, int64_t T, const void* W, bool w_bf16, int64_t N,
                                  int64_t K, float* xa, float* wa, int ncu, hipStream_t st) {
  if (x_bf16) {
    return w_bf16 ? col_absmax_pair_t<uint16_t, uint16_t>(X, T, W, N, K, xa, wa, ncu, st)
                  : col_absmax_pair_t<uint16_t, float>(X, T, W, N, K, xa, wa, ncu, st);
  }
  return w_bf16 ? col_absmax_pair_t<float, uint16_t>(X, T, W, N, K, xa, wa, ncu, st)
                : col_absmax_pair_t<float, float>(X, T, W, N, K, xa, wa, ncu, st);
}

hipError_t launch_col_absmax(const void* A, bool bf16, int64_t rows, int64_t cols, float* amax,
                             bool vec_ok, int ncu, hipStream_t st) {
  if (bf16) {
    const uint16_t* a = static_cast<const uint16_t*>(A);
    return vec_ok ? col_absmax_t<uint16_t, 8, 8>(a, rows, cols, amax, ncu, st)
                  : col_absmax_t<uint16_t, 1, 4>(a, rows, cols, amax, ncu, st);
  }
  const float* a = static_cast<const float*>(A);
  if (vec_ok) {
    const int64_t cb = (cols / 4 + 255) / 256;          // column blocks
    int64_t S = ncu / cb;                               // row interleave
    if (S < 1) S = 1;
    if (S > rows) S = rows;
    if (S > 65535) S = 65535;
    SQ_TRACE("col_absmax_blk (f32, 4 KB column blocks) rows %lld cols %lld, grid %lld blocks x %lld row interleave",
             (long long)rows, (long long)cols, (long long)cb, (long long)S);
    hipLaunchKernelGGL((col_absmax_blk_kernel<float, 8>), dim3((unsigned)cb, (unsigned)S), dim3(256), 0,
                       st, a, rows, cols, amax);
    return hipGetLastError();
  }
  return col_absmax_t<float, 1, 4>(a, rows, cols, amax, ncu, st);
}

template <typename T, int VEC, int U>
static hipError_t tensor_absmax_t(const T* A, int64_t rows, int64_t cols, const float* s, float* amax,
                                  int ncu, hipStream_t st) {
  const int64_t chunks = (cols + VEC - 1) / VEC;
  const int64_t gx = (chunks + 63) / 64;
  int64_t slabs = 8LL * ncu / gx;
  if (slabs < 1) slabs = 1;
  const int64_t max_slabs = (rows + 15) / 16;
  if (slabs > max_slabs) slabs = max_slabs;
  if (slabs > 65535) slabs = 65535;
  int64_t slab = (rows + slabs - 1) / slabs;
  slabs = (rows + slab - 1) / slab;
  const dim3 grid((unsigned)gx, (unsigned)slabs), block(256);
  SQ_TRACE("tensor_absmax (%s, slab form, %d elements per load) rows %lld cols %lld, grid %lld x %lld slabs",
           sizeof(T) == 2 ? "bf16" : "f32", VEC, (long long)rows, (long long)cols, (long long)gx, (long long)slabs);
  if (s) hipLaunchKernelGGL((tensor_absmax_kernel<T, VEC, U, true>), grid, block, 0, st, A, rows, cols, slab, s, amax);
  else hipLaunchKernelGGL((tensor_absmax_kernel<T, VEC, U, false>), grid, block, 0, st, A, rows, cols, slab, s, amax);
  return hipGetLastError();
}

// Row-walking range kernel: rows of K = 8 * 256 * CPT' elements (CPT' <= CPT).
// U rows in flight per group (about 16 / 32 loads of 16 bytes per thread for
// bf16 / fp32); one workgroup per CU for bf16, two for fp32 (measured best on
// 8192 x 8192: 24.6 us bf16, 48 us fp32, against 35 / 64 us for the slab form).
template <typename T, bool HAS_S, int CPT>
static hipError_t tensor_absmax_rows_t(const T* A, int64_t R, int64_t K, const float* s, float* amax,
                                       int ncu, hipStream_t st) {
  constexpr int U0 = (sizeof(T) == 2 ? 16 : 32) / CPT;
  constexpr int U = U0 > 16 ? 16 : U0;
  int64_t g = (R + U - 1) / U;
  const int64_t cap = (sizeof(T) == 2 ? 1 : 2) * (int64_t)ncu;
  if (g > cap) g = cap;
  SQ_TRACE("tensor_absmax_rows (%s, %d chunks of 8 per thread, %d rows per group) R %lld K %lld, grid %lld x 256 threads",
           sizeof(T) == 2 ? "bf16" : "f32", CPT, U, (long long)R, (long long)K, (long long)g);
  if (K == (int64_t)CPT * 2048)
    hipLaunchKernelGGL((tensor_absmax_rows_kernel<T, HAS_S, CPT, U, true>), dim3((unsigned)g), dim3(256), 0, st, A, R, K, s, amax);
  else
    hipLaunchKernelGGL((tensor_absmax_rows_kernel<T, HAS_S, CPT, U, false>), dim3((unsigned)g), dim3(256), 0, st, A, R, K, s, amax);
  return hipGetLastError();
}

template <typename T, bool HAS_S>
static hipError_t tensor_absmax_rows(const T* A, int64_t R, int64_t K, const float* s, float* amax,
                                     int ncu, hipStream_t st) {
  const int64_t cpt = (K / 8 + 255) / 256;
  if (cpt <= 1) return tensor_absmax_rows_t<T, HAS_S, 1>(A, R, K, s, amax, ncu, st);
  if (cpt <= 2) return tensor_absmax_rows_t<T, HAS_S, 2>(A, R, K, s, amax, ncu, st);
  if (cpt <= 4) return tensor_absmax_rows_t<T, HAS_S, 4>(A, R, K, s, amax, ncu, st);
  return tensor_absmax_rows_t<T, HAS_S, 8>(A, R, K, s, amax, ncu, st);
}

template <typename T>
static hipError_t tensor_absmax_any(const T* A, int64_t rows, int64_t cols, const float* s, float* amax,
                                    bool vec_ok, int ncu, hipStream_t st) {
  constexpr int VEC = 16 / sizeof(T);
  if (vec_ok && cols % 8 == 0 && cols <= 16384)
    return s ? tensor_absmax_rows<T, true>(A, rows, cols, s, amax, ncu, st)
             : tensor_absmax_rows<T, false>(A, rows, cols, s, amax, ncu, st);
  if (vec_ok) return tensor_absmax_t<T, VEC, (VEC == 8 ? 8 : 16)>(A, rows, cols, s, amax, ncu, st);
  return tensor_absmax_t<T, 1, 4>(A, rows, cols, s, amax, ncu, st);
}

hipError_t launch_tensor_absmax(const void* A, bool bf16, int64_t rows, int64_t cols, const float* s,
                                float* amax, bool vec_ok, int ncu, hipStream_t st) {
  if (bf16) return tensor_absmax_any(static_cast<const uint16_t*>(A), rows, cols, s, amax, vec_ok, ncu, st);
  return tensor_absmax_any(static_cast<const float*>(A), rows, cols, s, amax, vec_ok, ncu, st);
}

template <typename T>
static hipError_t smooth_from_w_t(const T* W, int64_t N, int64_t K, const float* xa, double alpha, float* s,
                                  bool vec_ok, hipStream_t st) {
  SQ_TRACE("smooth_w%s (%s, weight column maxima and factors in one pass) N %lld K %lld, alpha %g",
           vec_ok ? "strip" : "col", sizeof(T) == 2 ? "bf16" : "f32", (long long)N, (long long)K, alpha);
  if (vec_ok) {
    constexpr int SC = 8 * (16 / sizeof(T));
    hipLaunchKernelGGL((smooth_wstrip_kernel<T, 4>), dim3((unsigned)((K + SC - 1) / SC)), dim3(256), 0, st, W, N,
                       K, xa, alpha, s);
  } else {
    hipLaunchKernelGGL((smooth_wcol_kernel<T, 8>), dim3((unsigned)((K + 63) / 64)), dim3(256), 0, st, W, N, K,
                       xa, alpha, s);
  }
  return hipGetLastError();
}

hipError_t launch_smooth_scales_from_w(const void* W, bool bf16, int64_t N, int64_t K, const float* xa,
                                       float alpha, float* s, bool vec_ok, hipStream_t st) {
  if (bf16) return smooth_from_w_t(static_cast<const uint16_t*>(W), N, K, xa, (double)alpha, s, vec_ok, st);
  return smooth_from_w_t(static_cast<const float*>(W), N, K, xa, (double)alpha, s, vec_ok, st);
}

hipError_t launch_smooth_scales(const float* xa, const float* wa, int64_t K, float alpha, float* s,
                                hipStream_t st) {
  SQ_TRACE("smooth_scales K %lld, alpha %g", (long long)K, (double)alpha);
  hipLaunchKernelGGL(smooth_scales_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, xa,
                     wa, K, (double)alpha, s);
  return hipGetLastError();
}

}  // namespace sq
