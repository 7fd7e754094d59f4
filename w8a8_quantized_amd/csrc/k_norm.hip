// Normalisation fused with the smoothing and per-token int8 quantisation
// (gfx950): the producer in front of a W8A8 linear layer.
//
// multigrid.ai "SmoothQuant Explained", section "Why the rescaling is free at
// runtime": the smoothing division is folded offline into the gain of the norm
// that precedes the linear layer (gain / s, and bias / s for a LayerNorm), so the
// norm itself emits smoothed activations (inferenceinterviews.com "Why do
// activation outliers break INT8 W8A8...", section "A strong answer": 1/s_j folds
// into the preceding RMSNorm gain).  Here that norm also quantises its output
// per token, so the normalised activations never reach HBM: X is read once and
// only the int8 codes and scales are written.
//
//   RMSNorm   rstd = 1 / sqrt(mean_k x^2 + eps),                 h = (x * rstd) * g
//   LayerNorm mean = mean_k x, rstd = 1 / sqrt(mean_k (x - mean)^2 + eps),
//             h = ((x - mean) * rstd) * g + b
//   then scale = max_k |h| / 127 (1 for a zero row), code = clamp(rne(h / scale))
// The mean is summed in binary64; the (centred) squares are summed in binary32
// within each thread's 8-element chunks and in binary64 beyond (two passes for the
// variance, the row being in registers); each statistic is rounded once to
// binary32, within 1e-6 relative of a binary64 evaluation.  h is the binary32
// chain above, one rounding per operation.
//
// Fast path (row length a multiple of 8, at most 16384, 16-byte aligned rows):
// as the row quantiser, a workgroup of 4 waves walks rows blockIdx.x, +gridDim.x,
// ...; thread t owns the 8-element chunks t, t + 256, ... of a row, keeps the
// gains (and biases) of its columns in registers, holds the row in registers and
// has the next row's loads in flight.  Each reduction is a DPP wave reduction plus
// a 4-entry LDS exchange and one barrier (2 per row for RMSNorm, 3 for LayerNorm).
// Slow path: one workgroup per row, re-reading the row for each pass.
#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace sq {

// v + (v of the lane that DPP control CTRL names), for the rows in ROWM; lanes
// of other rows, and lanes without a source, add +0.  A binary64 value moves as
// its two 32-bit halves.
template <int CTRL, int ROWM>
__device__ __forceinline__ double dpp_add_f64(double v) {
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)u, CTRL, ROWM, 0xF, false);
  const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)(u >> 32), CTRL, ROWM, 0xF, false);
  return v + __builtin_bit_cast(double, ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo);
}

// Sum over the 64 lanes in binary64 (a fixed order); every lane gets the total.
// Pairs, quads, half rows and rows of 16 lanes combine through DPP, then rows 0+1
// and 2+3 (row_bcast15), then all four (row_bcast31) in lane 63, which is read
// back.  A butterfly of cross-lane shuffles in its place (each through the LDS
// crossbar) made the RMSNorm producer 3% and the LayerNorm producer 4% slower on
// 8192 x 8192 bf16, with identical statistics in every row.
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = dpp_add_f64<0xB1, 0xF>(v);    // quad_perm 1,0,3,2
  v = dpp_add_f64<0x4E, 0xF>(v);    // quad_perm 2,3,0,1
  v = dpp_add_f64<0x141, 0xF>(v);   // row_half_mirror
  v = dpp_add_f64<0x140, 0xF>(v);   // row_mirror
  v = dpp_add_f64<0x142, 0xA>(v);   // row_bcast15 into rows 1 and 3
  v = dpp_add_f64<0x143, 0xC>(v);   // row_bcast31 into rows 2 and 3
  const uint64_t u = __builtin_bit_cast(uint64_t, v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), 63);
  return __builtin_bit_cast(double, ((uint64_t)hi << 32) | (uint64_t)lo);
}

template <typename T> struct Row8;
template <> struct Row8<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void unpack(float* o) const {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  }
};
template <> struct Row8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = reinterpret_cast<const float4*>(p)[0];
    b = reinterpret_cast<const float4*>(p)[1];
  }
  __device__ __forceinline__ void zero() { a = b = make_float4(0.f, 0.f, 0.f, 0.f); }
  __device__ __forceinline__ void unpack(float* o) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

template <typename T, bool LAYER, bool HAS_B, int CPT, bool FULL>
__global__ __launch_bounds__(256) void norm_quant_rows_kernel(
    const T* __restrict__ A, int64_t R, int64_t K, const float* __restrict__ gain,
    const float* __restrict__ bias, float eps, int8_t* __restrict__ Q, float* __restrict__ scale_out,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
  __shared__ double red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nchunks = K >> 3;

  // gains and biases of this thread's columns (0 for chunks past the row end,
  // which makes their h exactly 0)
  float gv[CPT][8], bv[CPT][8];
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = (int64_t)j * 256 + tid;
    const bool ok = FULL || c < nchunks;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      gv[j][e] = ok ? gain[c * 8 + e] : 0.0f;
      bv[j][e] = (HAS_B && ok) ? bias[c * 8 + e] : 0.0f;
    }
  }

  // block-wide binary64 sum (or maximum of non-negative values); alternating
  // LDS slots, one barrier
  int par = 0;
  auto block_sum = [&](double v) {
    v = wave_sum_f64(v);
    if (lane == 0) red[par][wave] = v;
    __syncthreads();
    const double t = (red[par][0] + red[par][1]) + (red[par][2] + red[par][3]);
    par ^= 1;
    return t;
  };

  auto process = [&](const Row8<T>* raw, int64_t r) {
    float x[CPT][8];
#pragma unroll
    for (int j = 0; j < CPT; ++j) raw[j].unpack(x[j]);
    double mu = 0.0;
    if (LAYER) {
      double sum = 0.0;
#pragma unroll
      for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += (double)x[j][e];   // absent chunks hold 0
      mu = block_sum(sum) / (double)K;
    }
    // squares of each 8-element chunk summed in binary32 (non-negative terms: within
    // ~8 * 2^-24 relative), chunk sums added in binary64; measured ~10% faster
    // than binary64 throughout
    double ss = 0.0;
    const float muf = (float)mu;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = (int64_t)j * 256 + tid;
      if (FULL || c < nchunks) {
        float cs = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float d = LAYER ? x[j][e] - muf : x[j][e];
          cs = __builtin_fmaf(d, d, cs);
        }
        ss += (double)cs;
      }
    }
    const double var = block_sum(ss) / (double)K;
    const float rstd = (float)(1.0 / sqrt(var + (double)eps));
    const float mean = (float)mu;
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float cx = LAYER ? x[j][e] - mean : x[j][e];
        const float n = cx * rstd;
        float h = n * gv[j][e];
        if (HAS_B) h = h + bv[j][e];
        x[j][e] = h;
        m = fmaxf(m, fabsf(h));
      }
    m = wave_max_nonneg(m);
    if (lane == 0) red[par][wave] = (double)m;
    __syncthreads();
    const float amax = (float)fmax(fmax(red[par][0], red[par][1]), fmax(red[par][2], red[par][3]));
    par ^= 1;
    const float scale = amax == 0.0f ? 1.0f : amax / (float)kQmax;
    const double rsc = 1.0 / (double)scale;
    if (tid == 0) {
      scale_out[r] = scale;
      if (mean_out) mean_out[r] = mean;
      if (rstd_out) rstd_out[r] = rstd;
    }
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = (int64_t)j * 256 + tid;
      if (FULL || c < nchunks) {
        uint2 o;
        o.x = pack4_lowbytes(quant_code_bits(x[j][0], rsc), quant_code_bits(x[j][1], rsc),
                             quant_code_bits(x[j][2], rsc), quant_code_bits(x[j][3], rsc));
        o.y = pack4_lowbytes(quant_code_bits(x[j][4], rsc), quant_code_bits(x[j][5], rsc),
                             quant_code_bits(x[j][6], rsc), quant_code_bits(x[j][7], rsc));
        *reinterpret_cast<uint2*>(Q + r * K + c * 8) = o;
      }
    }
  };
  auto load = [&](Row8<T>* raw, int64_t r) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = (int64_t)j * 256 + tid;
      if (FULL || c < nchunks) raw[j].load(A + r * K + c * 8); else raw[j].zero();
    }
  };

  // Unconditional prefetch (past the last row it re-reads row R - 1, an L2
  // hit), held ahead of the row's arithmetic by a scheduling barrier: under a
  // branch the compiler waited for every outstanding load, the prefetch
  // included, before each row (RMSNorm 8192 x 8192 bf16: 37.4 against 39.4 us,
  // bit-identical).
  Row8<T> ba[CPT], bb[CPT];
  const int64_t G = gridDim.x;
  int64_t r = blockIdx.x;
  if (r >= R) return;
  load(ba, r);
  while (true) {
    load(bb, r + G < R ? r + G : R - 1);
    __builtin_amdgcn_sched_barrier(0);
    process(ba, r);
    r += G;
    if (r >= R) return;
    load(ba, r + G < R ? r + G : R - 1);
    __builtin_amdgcn_sched_barrier(0);
    process(bb, r);
    r += G;
    if (r >= R) return;
  }
}

// Any row length / alignment: one workgroup per row, one pass per statistic.
template <typename T> __device__ __forceinline__ float nload(const T* p);
template <> __device__ __forceinline__ float nload<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float nload<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T, bool LAYER>
__global__ __launch_bounds__(256) void norm_quant_rows_slow_kernel(
    const T* __restrict__ A, int64_t R, int64_t K, const float* __restrict__ gain,
    const float* __restrict__ bias, float eps, int8_t* __restrict__ Q, float* __restrict__ scale_out,
    float* __restrict__ mean_out, float* __restrict__ rstd_out) {
  __shared__ double red[4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto block_sum = [&](double v) {
    v = wave_sum_f64(v);
    if (lane == 0) red[wave] = v;
    __syncthreads();
    const double t = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return t;
  };
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* row = A + r * K;
    double mu = 0.0;
    if (LAYER) {
      double sum = 0.0;
      for (int64_t k = tid; k < K; k += 256) sum += (double)nload<T>(row + k);
      mu = block_sum(sum) / (double)K;
    }
    double ss = 0.0;
    for (int64_t k = tid; k < K; k += 256) {
      const double d = (double)nload<T>(row + k) - mu;
      ss += d * d;
    }
    const double var = block_sum(ss) / (double)K;
    const float rstd = (float)(1.0 / sqrt(var + (double)eps));
    const float mean = (float)mu;
    auto h_of = [&](int64_t k) {
      const float x = nload<T>(row + k);
      const float cx = LAYER ? x - mean : x;
      float h = (cx * rstd) * gain[k];
      if (LAYER && bias) h = h + bias[k];
      return h;
    };
    float m = 0.0f;
    for (int64_t k = tid; k < K; k += 256) m = fmaxf(m, fabsf(h_of(k)));
    m = wave_max(m);
    if (lane == 0) red[wave] = (double)m;
    __syncthreads();
    const float mx = (float)fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
    __syncthreads();
    const float scale = mx == 0.0f ? 1.0f : mx / (float)kQmax;
    if (tid == 0) {
      scale_out[r] = scale;
      if (mean_out) mean_out[r] = mean;
      if (rstd_out) rstd_out[r] = rstd;
    }
    for (int64_t k = tid; k < K; k += 256) {
      float q = __builtin_rintf(h_of(k) / scale);
      q = fminf(fmaxf(q, -(float)kQmax), (float)kQmax);
      Q[r * K + k] = (int8_t)(int)q;
    }
  }
}

template <typename T, bool LAYER, bool HAS_B>
static hipError_t norm_fast(const T* A, int64_t R, int64_t K, const float* g, const float* b, float eps,
                            int8_t* Q, float* sc, float* mean, float* rstd, int ncu, hipStream_t st) {
  const int cpt = (int)((K / 8 + 255) / 256);
  const int c2 = cpt <= 1 ? 1 : cpt <= 2 ? 2 : cpt <= 4 ? 4 : 8;
  const bool full = K == (int64_t)c2 * 2048;
  const int64_t g0 = R < 3LL * ncu ? R : 3LL * ncu;
  const dim3 grid((unsigned)g0), block(256);
  SQ_TRACE("norm_quant_rows (%s%s, %s) %d chunks of 8 per thread%s, R %lld K %lld, grid %lld x 256 threads",
           LAYER ? "LayerNorm" : "RMSNorm", HAS_B ? " with bias" : "", sizeof(T) == 2 ? "bf16" : "f32", c2,
           full ? ", full rows" : "", (long long)R, (long long)K, (long long)g0);
#define SQ_NORM_LAUNCH(C)                                                                                  \
  if (full) hipLaunchKernelGGL((norm_quant_rows_kernel<T, LAYER, HAS_B, C, true>), grid, block, 0, st, A, R, K, g, b, eps, Q, sc, mean, rstd); \
  else hipLaunchKernelGGL((norm_quant_rows_kernel<T, LAYER, HAS_B, C, false>), grid, block, 0, st, A, R, K, g, b, eps, Q, sc, mean, rstd);
  switch (c2) {
    case 1: SQ_NORM_LAUNCH(1) break;
    case 2: SQ_NORM_LAUNCH(2) break;
    case 4: SQ_NORM_LAUNCH(4) break;
    default: SQ_NORM_LAUNCH(8) break;
  }
#undef SQ_NORM_LAUNCH
  return hipGetLastError();
}

template <typename T>
static hipError_t norm_dispatch(const T* A, bool layer, int64_t R, int64_t K, const float* g, const float* b,
                                float eps, int8_t* Q, float* sc, float* mean, float* rstd, bool vec_ok, int ncu,
                                hipStream_t st) {
  if (vec_ok && K <= kQuantFastMaxK) {
    if (!layer) return norm_fast<T, false, false>(A, R, K, g, nullptr, eps, Q, sc, mean, rstd, ncu, st);
    return b ? norm_fast<T, true, true>(A, R, K, g, b, eps, Q, sc, mean, rstd, ncu, st)
             : norm_fast<T, true, false>(A, R, K, g, nullptr, eps, Q, sc, mean, rstd, ncu, st);
  }
  const int64_t g0 = R < 8LL * ncu ? R : 8LL * ncu;
  SQ_TRACE("norm_quant_rows_slow (%s, %s; K %% 8 != 0, unaligned rows or K > %lld) R %lld K %lld, grid %lld x 256 threads",
           layer ? "LayerNorm" : "RMSNorm", sizeof(T) == 2 ? "bf16" : "f32", (long long)kQuantFastMaxK, (long long)R,
           (long long)K, (long long)g0);
  if (layer)
    hipLaunchKernelGGL((norm_quant_rows_slow_kernel<T, true>), dim3((unsigned)g0), dim3(256), 0, st, A, R, K, g, b, eps, Q, sc, mean, rstd);
  else
    hipLaunchKernelGGL((norm_quant_rows_slow_kernel<T, false>), dim3((unsigned)g0), dim3(256), 0, st, A, R, K, g, b, eps, Q, sc, mean, rstd);
  return hipGetLastError();
}

hipError_t launch_norm_quant(const void* A, bool bf16, bool layer, int64_t R, int64_t K, const float* gain,
                             const float* bias, float eps, int8_t* Q, float* scale, float* mean, float* rstd,
                             bool vec_ok, int ncu, hipStream_t st) {
  if (bf16)
    return norm_dispatch(static_cast<const uint16_t*>(A), layer, R, K, gain, bias, eps, Q, scale, mean, rstd, vec_ok, ncu, st);
  return norm_dispatch(static_cast<const float*>(A), layer, R, K, gain, bias, eps, Q, scale, mean, rstd, vec_ok, ncu, st);
}

__global__ void fold_gain_kernel(const float* __restrict__ v, const float* __restrict__ s, int64_t K,
                                 float* __restrict__ out) {
  const int64_t k = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (k < K) out[k] = v[k] / s[k];
}

hipError_t launch_fold_gain(const float* v, const float* s, int64_t K, float* out, hipStream_t st) {
  SQ_TRACE("fold_gain K %lld", (long long)K);
  hipLaunchKernelGGL(fold_gain_kernel, dim3((unsigned)((K + 255) / 256)), dim3(256), 0, st, v, s, K, out);
  return hipGetLastError();
}

}  // namespace sq
