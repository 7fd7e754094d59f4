// Row quantisers (gfx950): dynamic per-token activation quantisation fused with
// the smoothing division, and per-output-channel weight quantisation fused with
// the smoothing multiply.
//
// Both are the symmetric int8 round trip of maitreyasuin.github.io
// "...01-one-outlier", section "The four operations" (scale = amax / 127, code =
// clamp(round(v / scale), -127, 127), an all-zero row gets scale 1 and codes 0),
// applied per row of X diag(s)^-1 (tokens) or of W diag(s) (output channels)
// as on inferenceinterviews.com "Why do activation outliers break INT8 W8A8...",
// section "A strong answer".
//
// Fast path (row length a multiple of 8, 16-byte aligned rows): a workgroup of 4
// waves owns a fixed set of 8-element column chunks (chunk c = j*256 + thread)
// and walks rows r = blockIdx.x, blockIdx.x + gridDim.x, ...  Per-column factors
// (the binary64 reciprocal of s for the division, or s itself for the multiply)
// therefore stay in registers across all of the workgroup's rows.  Each row is
// read from HBM once, held in registers, reduced to its absmax (DPP wave
// reduction + a 4-entry LDS exchange, one barrier), then turned into codes and written with
// 8-byte stores.  The next row's loads are issued before the current row is
// processed.  Both divisions of the method are done exactly as a multiply by a
// binary64 reciprocal (see div_by_recip).
//
// Static-range mode (MODE 2, per-tensor activation scales): the range is given
// (a calibrated clip, or the tensor's own range found by a reduction launched
// before), so scale = clip / 127 is known up front and a row needs no reduction
// and no barrier: read, divide, quantise, store (maitreyasuin page, "The four
// operations", quantize_dequantize with its clip argument; clip = 0 gives scale 1
// and codes 0).
//
// FP8 mode (F8): the same round trip on the E4M3 grid (inferenceinterviews.com,
// formats paragraph: per-token FP8 activations): scale = amax / 448, code = the
// E4M3 value nearest to v / scale (ties to even), saturated at +-448; the exact
// binary32 quotient goes through the hardware conversion (see e4m3_pack4).
//
// The multiply mode (MODE 1) also serves the mixed-precision decomposition's
// bulk rows, weights and activations alike, with s a 0/1 column mask.  Weight
// codes (NTS) are written with non-temporal stores, activation codes with
// ordinary ones.
//
// Slow path (any shape/alignment): one workgroup per row, two passes over the
// row with plain IEEE binary32 divisions; identical results.
#include "common.h"
#include "kernels.h"
#include "trace.h"

namespace sq {

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// 8 consecutive elements of one row as raw bits.
template <typename T> struct Raw8;
template <> struct Raw8<uint16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const uint16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void zero() { v = make_uint4(0, 0, 0, 0); }
  __device__ __forceinline__ void unpack(float* o) const {
    o[0] = bf16_lo(v.x); o[1] = bf16_hi(v.x); o[2] = bf16_lo(v.y); o[3] = bf16_hi(v.y);
    o[4] = bf16_lo(v.z); o[5] = bf16_hi(v.z); o[6] = bf16_lo(v.w); o[7] = bf16_hi(v.w);
  }
};
template <> struct Raw8<float> {
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

// Binary64 reciprocal accurate to ~1 ulp: hardware estimate + two Newton steps.
// (The exactness argument of div_by_recip needs only a relative error < 2^-50.)
__device__ __forceinline__ double recip64(double b) {
  double y = __builtin_amdgcn_rcp(b);
  double e = __builtin_fma(-b, y, 1.0);
  y = __builtin_fma(y, e, y);
  e = __builtin_fma(-b, y, 1.0);
  return __builtin_fma(y, e, y);
}

// Static-range scale: clip / 127, or 1 (with a zero reciprocal, so that every
// code is 0) when the range is 0.
__device__ __forceinline__ void static_scale(const float* clip, float& scale, double& rscale) {
  const float c = *clip;
  scale = c == 0.0f ? 1.0f : c / (float)kQmax;
  rscale = c == 0.0f ? 0.0 : 1.0 / (double)scale;
}

constexpr const char* kQuantModeName[3] = {"activations, per-row range", "multiply by s, per-row range",
                                           "activations, given range"};

// MODE: 0 = activations, per-row range (divide by s); 1 = weights, per-row range
// (multiply by s); 2 = activations, given range *clip (divide by s).
// FULL: K == CPT * 2048, every thread's chunks exist (no per-chunk masks).
// F8: E4M3 codes (MODE 0 or 1) instead of int8.  NTS: non-temporal code stores.
template <typename T, int MODE, bool HAS_S, int CPT, bool FULL, bool F8, bool NTS>
__global__ __launch_bounds__(256) void quant_rows_kernel(const T* __restrict__ A, int64_t R,
                                                         int64_t K, const float* __restrict__ s,
                                                         const float* __restrict__ clip,
                                                         int8_t* __restrict__ Q,
                                                         float* __restrict__ scale_out) {
  __shared__ float red[2][4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t nchunks = K >> 3;
  constexpr bool kDivide = MODE != 1;
  float s_scale = 1.0f;
  double s_rscale = 0.0;
  if (MODE == 2) static_scale(clip, s_scale, s_rscale);

  // per-column factors for the chunks this thread owns
  double rs[CPT][8];   // MODE 0, 2: 1 / s
  float sv[CPT][8];    // MODE 1: s
#pragma unroll
  for (int j = 0; j < CPT; ++j) {
    const int64_t c = (int64_t)j * 256 + tid;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float f = 1.0f;
      if (HAS_S && (FULL || c < nchunks)) f = s[c * 8 + e];
      if (kDivide) rs[j][e] = HAS_S ? recip64((double)f) : 1.0;
      else sv[j][e] = f;
    }
  }

  // one row: smoothed values, row maximum (wave DPP reduction + 4-entry LDS
  // exchange) unless the range is given, scale, codes
  int par = 0;
  auto process = [&](const Raw8<T>* raw, int64_t r) {
    float v[CPT][8];
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      float x[8];
      raw[j].unpack(x);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        float h = x[e];
        if (HAS_S) h = kDivide ? div_by_recip(x[e], rs[j][e]) : x[e] * sv[j][e];
        v[j][e] = h;
        m = fmaxf(m, fabsf(h));
      }
    }
    float scale = s_scale;
    double rsc = s_rscale;
    if (MODE != 2) {
      m = wave_max_nonneg(m);
      if (lane == 0) red[par][wave] = m;
      __syncthreads();
      const float amax = fmaxf(fmaxf(red[par][0], red[par][1]), fmaxf(red[par][2], red[par][3]));
      par ^= 1;
      scale = amax == 0.0f ? 1.0f : amax / (F8 ? kF8max : (float)kQmax);
      rsc = amax == 0.0f ? 0.0 : 1.0 / (double)scale;   // a zero row: every code 0
    }
    if (tid == 0) scale_out[r] = scale;
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = (int64_t)j * 256 + tid;
      if (FULL || c < nchunks) {
        uint2 o;
        if (F8) {
          // exact quotients, then the E4M3 conversion; a zero row (rsc = 0) is
          // written as zero codes
          float q[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) q[e] = div_by_recip(v[j][e], rsc);
          o.x = rsc == 0.0 ? 0u : e4m3_pack4(q[0], q[1], q[2], q[3]);
          o.y = rsc == 0.0 ? 0u : e4m3_pack4(q[4], q[5], q[6], q[7]);
        } else {
          o.x = pack4_lowbytes(quant_code_bits(v[j][0], rsc), quant_code_bits(v[j][1], rsc),
                               quant_code_bits(v[j][2], rsc), quant_code_bits(v[j][3], rsc));
          o.y = pack4_lowbytes(quant_code_bits(v[j][4], rsc), quant_code_bits(v[j][5], rsc),
                               quant_code_bits(v[j][6], rsc), quant_code_bits(v[j][7], rsc));
        }
        if constexpr (NTS) {
          // weight codes are read back much later: non-temporal stores
          // (8192 x 8192 fp32 weights 5% faster; activation codes, read by the
          // GEMM right after, were slower this way)
          u32x2 ov;
          ov[0] = o.x;
          ov[1] = o.y;
          __builtin_nontemporal_store(ov, reinterpret_cast<u32x2*>(Q + r * K + c * 8));
        } else {
          *reinterpret_cast<uint2*>(Q + r * K + c * 8) = o;
        }
      }
    }
  };
  auto load = [&](Raw8<T>* raw, int64_t r) {
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
      const int64_t c = (int64_t)j * 256 + tid;
      if (FULL || c < nchunks) raw[j].load(A + r * K + c * 8); else raw[j].zero();
    }
  };

  // rows r, r + G, r + 2G, ... alternating between two register buffers; the
  // next row's loads are in flight while the current one is processed.  The
  // prefetch is unconditional (past the last row it re-reads row R - 1, an L2
  // hit) and held ahead of the row's arithmetic by a scheduling barrier: a
  // prefetch under a branch made the compiler wait for every outstanding load
  // (the prefetch included) before each row, and the weight quantiser ran 3%
  // slower that way (8192 x 8192 fp32, bit-identical).
  Raw8<T> ba[CPT], bb[CPT];
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

// Any row length / alignment: one workgroup per row, plain binary32 divisions.
template <typename T> __device__ __forceinline__ float load1(const T* p);
template <> __device__ __forceinline__ float load1<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T, int MODE, bool F8>
__global__ __launch_bounds__(256) void quant_rows_slow_kernel(const T* __restrict__ A, int64_t R,
                                                              int64_t K, const float* __restrict__ s,
                                                              const float* __restrict__ clip,
                                                              int8_t* __restrict__ Q,
                                                              float* __restrict__ scale_out) {
  __shared__ float red[4];
  const int tid = threadIdx.x;
  const float c = MODE == 2 ? *clip : 0.0f;
  for (int64_t r = blockIdx.x; r < R; r += gridDim.x) {
    const T* row = A + r * K;
    float scale;
    bool zero;
    if (MODE == 2) {
      zero = c == 0.0f;
      scale = zero ? 1.0f : c / (float)kQmax;
    } else {
      float m = 0.0f;
      for (int64_t k = tid; k < K; k += 256) {
        float x = load1<T>(row + k);
        if (s) x = (MODE == 1) ? x * s[k] : x / s[k];
        m = fmaxf(m, fabsf(x));
      }
      m = wave_max(m);
      if ((tid & 63) == 0) red[tid >> 6] = m;
      __syncthreads();
      const float amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
      __syncthreads();
      zero = amax == 0.0f;
      scale = zero ? 1.0f : amax / (F8 ? kF8max : (float)kQmax);
    }
    if (tid == 0) scale_out[r] = scale;
    for (int64_t k = tid; k < K; k += 256) {
      float x = load1<T>(row + k);
      if (s) x = (MODE == 1) ? x * s[k] : x / s[k];
      if (F8) {
        Q[r * K + k] = (int8_t)(zero ? 0u : e4m3_code(x / scale));
        continue;
      }
      float q = zero ? 0.0f : __builtin_rintf(x / scale);
      q = fminf(fmaxf(q, -(float)kQmax), (float)kQmax);
      Q[r * K + k] = (int8_t)(int)q;
    }
  }
}

template <typename T, int MODE, bool HAS_S, bool F8, bool NTS>
static hipError_t quant_fast(const T* A, int64_t R, int64_t K, const float* s, const float* clip,
                             int8_t* Q, float* scale, int ncu, hipStream_t st) {
  const int64_t nchunks = K / 8;
  const int cpt = (int)((nchunks + 255) / 256);
  int64_t g = R < 3LL * ncu ? R : 3LL * ncu;
  dim3 grid((unsigned)g), block(256);
  const int c2 = cpt <= 1 ? 1 : cpt <= 2 ? 2 : cpt <= 4 ? 4 : 8;   // instantiated sizes
  const bool full = K == (int64_t)c2 * 2048;
  SQ_TRACE("quant_rows (%s%s%s, %s) %d chunks of 8 per thread%s, R %lld K %lld, grid %lld x 256 threads",
           kQuantModeName[MODE], HAS_S ? ", smoothing" : "", F8 ? ", fp8" : "", sizeof(T) == 2 ? "bf16" : "f32", c2,
           full ? ", full rows" : "", (long long)R, (long long)K, (long long)g);
#define SQ_QUANT_LAUNCH(C)                                                                              \
  if (full) hipLaunchKernelGGL((quant_rows_kernel<T, MODE, HAS_S, C, true, F8, NTS>), grid, block, 0, st, A, R, K, s, clip, Q, scale); \
  else hipLaunchKernelGGL((quant_rows_kernel<T, MODE, HAS_S, C, false, F8, NTS>), grid, block, 0, st, A, R, K, s, clip, Q, scale);
  switch (c2) {
    case 1: SQ_QUANT_LAUNCH(1) break;
    case 2: SQ_QUANT_LAUNCH(2) break;
    case 4: SQ_QUANT_LAUNCH(4) break;
    default: SQ_QUANT_LAUNCH(8) break;
  }
#undef SQ_QUANT_LAUNCH
  return hipGetLastError();
}

template <typename T, int MODE, bool F8 = false, bool NTS = false>
static hipError_t quant_dispatch(const T* A, int64_t R, int64_t K, const float* s, const float* clip,
                                 int8_t* Q, float* scale, bool vec_ok, int ncu, hipStream_t st) {
  if (vec_ok && K <= kQuantFastMaxK) {
    return s ? quant_fast<T, MODE, true, F8, NTS>(A, R, K, s, clip, Q, scale, ncu, st)
             : quant_fast<T, MODE, false, F8, NTS>(A, R, K, s, clip, Q, scale, ncu, st);
  }
  int64_t g = R < 8LL * ncu ? R : 8LL * ncu;
  SQ_TRACE("quant_rows_slow (%s%s%s, %s; K %% 8 != 0, unaligned rows or K > %lld) R %lld K %lld, grid %lld x 256 threads",
           kQuantModeName[MODE], s ? ", smoothing" : "", F8 ? ", fp8" : "", sizeof(T) == 2 ? "bf16" : "f32",
           (long long)kQuantFastMaxK, (long long)R, (long long)K, (long long)g);
  hipLaunchKernelGGL((quant_rows_slow_kernel<T, MODE, F8>), dim3((unsigned)g), dim3(256), 0, st, A, R, K,
                     s, clip, Q, scale);
  return hipGetLastError();
}

template <typename T>
static hipError_t quant_mode(const T* A, int mode, int64_t R, int64_t K, const float* s,
                             const float* clip, int8_t* Q, float* scale, bool vec_ok, int ncu,
                             hipStream_t st) {
  switch (mode) {
    case kQuantWeights: return quant_dispatch<T, 1, false, true>(A, R, K, s, clip, Q, scale, vec_ok, ncu, st);
    case kQuantActMasked: return quant_dispatch<T, 1>(A, R, K, s, clip, Q, scale, vec_ok, ncu, st);
    case kQuantActStatic: return quant_dispatch<T, 2>(A, R, K, s, clip, Q, scale, vec_ok, ncu, st);
    case kQuantActF8: return quant_dispatch<T, 0, true>(A, R, K, s, clip, Q, scale, vec_ok, ncu, st);
    case kQuantWeightsF8: return quant_dispatch<T, 1, true, true>(A, R, K, s, clip, Q, scale, vec_ok, ncu, st);
    default: return quant_dispatch<T, 0>(A, R, K, s, clip, Q, scale, vec_ok, ncu, st);
  }
}

hipError_t launch_quant_rows(const void* A, bool bf16, int mode, int64_t R, int64_t K,
                             const float* s, const float* clip, int8_t* Q, float* scale,
                             bool vec_ok, int ncu, hipStream_t st) {
  if (bf16) return quant_mode(static_cast<const uint16_t*>(A), mode, R, K, s, clip, Q, scale, vec_ok, ncu, st);
  return quant_mode(static_cast<const float*>(A), mode, R, K, s, clip, Q, scale, vec_ok, ncu, st);
}

}  // namespace sq
