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

namespace sq {

// mask[j] = 0 when column j is among the n_o columns with the largest absmax
// (ties to the lower index), else 1.  rank_j = #{i : a_i > a_j or (a_i == a_j and
// i < j)}; each workgroup stages tiles of the vector in LDS.
__global__ __launch_bounds__(256) void decomp_rank_kernel(const float* __restrict__ a, int64_t K,
                                                          int64_t n_o, float* __restrict__ mask) {
  __shared__ float tile[256];
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const float aj = j < K ? a[j] : 0.0f;
  int64_t rank = 0;
  for (int64_t i0 = 0; i0 < K; i0 += 256) {
    __syncthreads();
    tile[threadIdx.x] = i0 + threadIdx.x < K ? a[i0 + threadIdx.x] : 0.0f;
    __syncthreads();
    const int lim = K - i0 < 256 ? (int)(K - i0) : 256;
    for (int u = 0; u < lim; ++u) {
      const float ai = tile[u];
      rank += (ai > aj) || (ai == aj && i0 + u < j);
    }
  }
  if (j < K) mask[j] = rank < n_o ? 0.0f : 1.0f;
}

// idx[p] = the p-th column (ascending) whose mask is 0.
__global__ __launch_bounds__(256) void decomp_index_kernel(const float* __restrict__ mask, int64_t K,
                                                           int32_t* __restrict__ idx) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= K || mask[j] != 0.0f) return;
  int64_t p = 0;
  for (int64_t i = 0; i < j; ++i) p += mask[i] == 0.0f;
  idx[p] = (int32_t)j;
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
  const dim3 grid((unsigned)((K + 255) / 256)), block(256);
  hipLaunchKernelGGL(decomp_rank_kernel, grid, block, 0, st, absmax, K, n_o, mask);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || n_o == 0) return e;
  hipLaunchKernelGGL(decomp_index_kernel, grid, block, 0, st, mask, K, idx);
  return hipGetLastError();
}

hipError_t launch_decomp_gather(const void* A, bool bf16, int64_t rows, int64_t K, const int32_t* idx,
                                int64_t n_o, float* out, int ncu, hipStream_t st) {
  const int64_t total = rows * n_o;
  if (total == 0) return hipSuccess;
  int64_t g = (total + 255) / 256;
  if (g > 8LL * ncu) g = 8LL * ncu;
  if (bf16)
    hipLaunchKernelGGL(decomp_gather_kernel<uint16_t>, dim3((unsigned)g), dim3(256), 0, st,
                       static_cast<const uint16_t*>(A), rows, K, idx, n_o, out);
  else
    hipLaunchKernelGGL(decomp_gather_kernel<float>, dim3((unsigned)g), dim3(256), 0, st,
                       static_cast<const float*>(A), rows, K, idx, n_o, out);
  return hipGetLastError();
}

}  // namespace sq
