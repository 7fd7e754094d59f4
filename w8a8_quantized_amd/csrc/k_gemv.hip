// Decode-shaped W8A8 GEMM (few tokens, T <= 64) on gfx950.
//
// With a handful of tokens the layer is bound by streaming the int8 weights from
// HBM (multigrid.ai "SmoothQuant Explained", section "Where it fits": at small
// batch the multiply is not the bottleneck).  Every weight byte is used by all T
// tokens at once, so there is no reuse to stage through LDS: each weight row
// segment goes straight from HBM into MFMA operand registers.
//
// v_mfma_i32_16x16x64_i8 takes a 16-row block of Wq as operand A (rows = output
// channels) and a 16-token block of Xq as operand B.  A lane supplies 16
// consecutive bytes of one row; the 4 lane groups cover 64 consecutive bytes, so
// one load instruction per operand reads 64 contiguous bytes of 16 rows.  Four
// such MFMAs cover a 256-byte K block.  The 4 waves of a workgroup split K
// (wave w takes blocks w, w+4, ...), and their int32 partial sums meet in LDS
// (integer addition: exact, order-free).  The epilogue is the one of the prefill
// kernel: y = fl32(fl32(acc) * fl32(x_scale[t] * w_scale[n])).
#include "common.h"
#include "kernels.h"

namespace sq {

template <int NB, int TB, int OUT>
__global__ __launch_bounds__(256) void gemv_i8_mfma_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ xs, const int8_t* __restrict__ Wq,
    const float* __restrict__ ws, int64_t T, int64_t N, int64_t K, void* __restrict__ Y,
    int vec_store) {
  __shared__ v4i red[4][NB * TB][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, grp = lane >> 4;
  const int64_t n0 = (int64_t)blockIdx.x * (NB * 16);

  const int8_t* wrow[NB];
  const int8_t* xrow[TB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    int64_t n = n0 + i * 16 + r16; n = n < N ? n : N - 1;   // clamped rows are never stored
    wrow[i] = Wq + n * K + grp * 16;
  }
#pragma unroll
  for (int b = 0; b < TB; ++b) {
    int64_t t = b * 16 + r16; t = t < T ? t : T - 1;
    xrow[b] = Xq + t * K + grp * 16;
  }

  v4i acc[NB][TB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[i][b] = v4i{0, 0, 0, 0};

  const int64_t nkb = (K + 255) / 256;

  for (int64_t kb = wave; kb < nkb; kb += 4) {
    const int64_t k = kb * 256;
    v4i wv[NB][4], xv[TB][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t off = k + j * 64;
      const bool ok = off + grp * 16 < K;
#pragma unroll
      for (int i = 0; i < NB; ++i)
        wv[i][j] = ok ? *reinterpret_cast<const v4i*>(wrow[i] + off) : v4i{0, 0, 0, 0};
#pragma unroll
      for (int b = 0; b < TB; ++b)
        xv[b][j] = ok ? *reinterpret_cast<const v4i*>(xrow[b] + off) : v4i{0, 0, 0, 0};
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int b = 0; b < TB; ++b)
          acc[i][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv[i][j], xv[b][j], acc[i][b], 0, 0, 0);
  }

#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int b = 0; b < TB; ++b) red[wave][i * TB + b][lane] = acc[i][b];
  __syncthreads();

  // wave w finishes blocks p = w, w+4, ...; lane holds n = n0 + i*16 + 4*grp + 0..3, t = b*16 + r16
  for (int p = wave; p < NB * TB; p += 4) {
    const int i = p / TB, b = p % TB;
    const v4i s0 = red[0][p][lane], s1 = red[1][p][lane], s2 = red[2][p][lane], s3 = red[3][p][lane];
    const int a4[4] = {s0[0] + s1[0] + s2[0] + s3[0], s0[1] + s1[1] + s2[1] + s3[1],
                       s0[2] + s1[2] + s2[2] + s3[2], s0[3] + s1[3] + s2[3] + s3[3]};
    const int64_t t = b * 16 + r16;
    const int64_t n = n0 + i * 16 + 4 * grp;
    if (t >= T || n >= N) continue;
    const int64_t nrem = N - n;
    const bool vec = vec_store && nrem >= 4;
    if (OUT == kOutI32) {
      int* y = static_cast<int*>(Y) + t * N + n;
      if (vec) *reinterpret_cast<int4*>(y) = make_int4(a4[0], a4[1], a4[2], a4[3]);
      else for (int e = 0; e < 4 && e < nrem; ++e) y[e] = a4[e];
      continue;
    }
    const float sc = xs[t];
    float v[4];
    for (int e = 0; e < 4; ++e) v[e] = (e < nrem) ? (float)a4[e] * (sc * ws[n + e]) : 0.0f;
    if (OUT == kOutF32) {
      float* y = static_cast<float*>(Y) + t * N + n;
      if (vec) *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
      else for (int e = 0; e < 4 && e < nrem; ++e) y[e] = v[e];
    } else {
      uint16_t* y = static_cast<uint16_t*>(Y) + t * N + n;
      if (vec) {
        uint2 pk;
        pk.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
        pk.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<uint2*>(y) = pk;
      } else {
        for (int e = 0; e < 4 && e < nrem; ++e) y[e] = (uint16_t)f32_to_bf16(v[e]);
      }
    }
  }
}

template <int NB, int TB>
static hipError_t gemv_cfg(const GemmArgs& a, hipStream_t st) {
  const int64_t G = (a.N + NB * 16 - 1) / (NB * 16);
  dim3 grid((unsigned)G), block(256);
  const int vs = a.vec_store ? 1 : 0;
  switch (a.out) {
    case kOutF32:
      hipLaunchKernelGGL((gemv_i8_mfma_kernel<NB, TB, kOutF32>), grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y, vs);
      break;
    case kOutBF16:
      hipLaunchKernelGGL((gemv_i8_mfma_kernel<NB, TB, kOutBF16>), grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y, vs);
      break;
    default:
      hipLaunchKernelGGL((gemv_i8_mfma_kernel<NB, TB, kOutI32>), grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y, vs);
      break;
  }
  return hipGetLastError();
}

hipError_t launch_gemv_mfma(const GemmArgs& a, int ncu, hipStream_t st) {
  (void)ncu;
  if (a.T <= 16) return gemv_cfg<2, 1>(a, st);
  if (a.T <= 32) return gemv_cfg<2, 2>(a, st);
  return gemv_cfg<2, 4>(a, st);
}

}  // namespace sq
