// Mixed-precision decomposition support (gfx950): choosing the static outlier
// channel set and gathering the outlier columns.
//
// mercemay.com "Activation Outlier Channels and Mixed-Precision Decomposition",
// section "Decomposition: keep the outliers in high precision": the contraction
// splits into the bulk channels, multiplied in int8, and a few outlier channels
// multiplied in floating point; the outlier set is determined once from
// calibration and stored with the weights.  maitreyasuin.github.io
// "...01-one-outlier", section "Route it, or move it": the outlier dimensions are
// the ones with the largest maximum magnitude.
//
// The int8 side needs no compaction: the bulk operands keep their full width
// with the outlier columns zeroed (the row quantiser multiplies by a 0/1 column
// mask), so the unchanged GEMM main loop sums exactly the bulk products and the
// per-token / per-channel bulk scales ignore the outliers.  The outlier columns
// are gathered in binary32, stored outlier-major ([n_o][rows]) so that the GEMM
// epilogue reads four consecutive channels, or a wave's tokens, with one access.
#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace sq {

// mask[j] = 0 when column j is among the n_o columns with the largest absmax
// (ties to the lower index), else 1.  rank_j = #{i : a_i > a_j or (a_i == a_j and
// i < j)}, a permutation of 0..K-1.  A workgroup owns 64 columns j (one per lane);
// its four waves split each 1024-value LDS tile of the vector in quarters and read
// it four values at a time; the four partial counts meet in LDS.  Tile entries
// past K hold -inf at indices >= K > j, so they never count.
__global__ __launch_bounds__(256) void decomp_rank_kernel(const float* __restrict__ a, int64_t K,
                                                          int64_t n_o, float* __restrict__ mask) {
  __shared__ float4 tile[256];
  __shared__ int part[4][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t j = (int64_t)blockIdx.x * 64 + lane;
  const float aj = j < K ? a[j] : 0.0f;
  int rank = 0;
  for (int64_t i0 = 0; i0 < K; i0 += 1024) {
    __syncthreads();
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t i = i0 + 4 * threadIdx.x + e;
      v[e] = i < K ? a[i] : -__builtin_inff();
    }
    tile[threadIdx.x] = make_float4(v[0], v[1], v[2], v[3]);
    __syncthreads();
    const int64_t left = K - i0 - 256 * wave;   // values of this wave's quarter that exist
    const int nq = left <= 0 ? 0 : (left >= 256 ? 64 : (int)((left + 3) / 4));
    for (int q = 0; q < nq; ++q) {
      const float4 t = tile[wave * 64 + q];
      const int64_t ib = i0 + 256 * wave + 4 * q;
      rank += (t.x > aj) || (t.x == aj && ib < j);
      rank += (t.y > aj) || (t.y == aj && ib + 1 < j);
      rank += (t.z > aj) || (t.z == aj && ib + 2 < j);
      rank += (t.w > aj) || (t.w == aj && ib + 3 < j);
    }
  }
  part[wave][lane] = rank;
  __syncthreads();
  if (wave == 0 && j < K) {
    const int r = part[0][lane] + part[1][lane] + part[2][lane] + part[3][lane];
    mask[j] = r < n_o ? 0.0f : 1.0f;
  }
}

// idx[p] = the p-th column (ascending) whose mask is 0.  One workgroup: each
// thread counts the zeros of its contiguous share of the mask, an exclusive scan
// of the counts in LDS gives each share's first position, and each thread writes
// the indices of its share's zeros.  Positions past n_o are not written (the
// mask has exactly n_o zeros unless the absmax vector holds a NaN).
__global__ __launch_bounds__(1024) void decomp_index_kernel(const float* __restrict__ mask, int64_t K,
                                                            int64_t n_o, int32_t* __restrict__ idx) {
  __shared__ int cnt[1024];
  const int t = threadIdx.x;
  const int64_t per = (K + 1023) / 1024;
  const int64_t b = t * per < K ? t * per : K;
  const int64_t e = b + per < K ? b + per : K;
  int c = 0;
  for (int64_t i = b; i < e; ++i) c += mask[i] == 0.0f;
  cnt[t] = c;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int add = t >= off ? cnt[t - off] : 0;
    __syncthreads();
    cnt[t] += add;
    __syncthreads();
  }
  int64_t p = cnt[t] - c;
  for (int64_t i = b; i < e; ++i)
    if (mask[i] == 0.0f) {
      if (p < n_o) idx[p] = (int32_t)i;
      ++p;
    }
}

template <typename T> __device__ __forceinline__ float gload(const T* p);
template <> __device__ __forceinline__ float gload<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float gload<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// out[o][r] = A[r][idx[o]] in binary32 (bf16 widened exactly); an index outside
// [0, K) gives a zero column instead of an out-of-range read.
template <typename T>
__global__ __launch_bounds__(256) void decomp_gather_kernel(const T* __restrict__ A, int64_t rows, int64_t K,
                                                            const int32_t* __restrict__ idx, int64_t n_o,
                                                            float* __restrict__ out) {
  const int64_t total = rows * n_o;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total; e += (int64_t)gridDim.x * 256) {
    const int64_t o = e / rows, r = e - o * rows;
    const int64_t k = idx[o];
    out[e] = (k >= 0 && k < K) ? gload<T>(A + r * K + k) : 0.0f;
  }
}

hipError_t launch_decomp_select(const float* absmax, int64_t K, int64_t n_o, int32_t* idx, float* mask,
                                hipStream_t st) {
  SQ_TRACE("decomp_rank + decomp_index (outlier set: %lld of K %lld columns)", (long long)n_o, (long long)K);
  hipLaunchKernelGGL(decomp_rank_kernel, dim3((unsigned)((K + 63) / 64)), dim3(256), 0, st, absmax, K, n_o, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_o == 0) return e;
  hipLaunchKernelGGL(decomp_index_kernel, dim3(1), dim3(1024), 0, st, mask, K, n_o, idx);
  return hipGetLastError();
}

hipError_t launch_decomp_gather(const void* A, bool bf16, int64_t rows, int64_t K, const int32_t* idx,
                                int64_t n_o, float* out, int ncu, hipStream_t st) {
  const int64_t total = rows * n_o;
  if (total == 0) return hipSuccess;
  int64_t g = (total + 255) / 256;
  if (g > 8LL * ncu) g = 8LL * ncu;
  SQ_TRACE("decomp_gather (%s) %lld outlier columns of %lld rows, K %lld, grid %lld x 256 threads",
           bf16 ? "bf16" : "f32", (long long)n_o, (long long)rows, (long long)K, (long long)g);
  if (bf16)
    hipLaunchKernelGGL(decomp_gather_kernel<uint16_t>, dim3((unsigned)g), dim3(256), 0, st,
                       static_cast<const uint16_t*>(A), rows, K, idx, n_o, out);
  else
    hipLaunchKernelGGL(decomp_gather_kernel<float>, dim3((unsigned)g), dim3(256), 0, st,
                       static_cast<const float*>(A), rows, K, idx, n_o, out);
  return hipGetLastError();
}

}  // namespace sq
