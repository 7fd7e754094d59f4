// W8A8 GEMM with int32 accumulation and the dequantising epilogue (gfx950).
//
//   acc[t][n] = sum_k Xq[t][k] * Wq[n][k]                        (exact int32)
//   Y[t][n]   = fl32(fl32(acc) * fl32(x_scale[t] * w_scale[n]))   (F32 / BF16 out)
// The per-token and per-output-channel scales factor out of the sum
// (maitreyasuin.github.io "...01-one-outlier", section "Which scales factor out,
// and why"), so the main loop is a plain integer contraction and the scales are
// applied once in the epilogue (mercemay.com "Activation Outlier Channels...",
// section "Decomposition": integer matmul, float epilogue).
//
// Prefill kernel: v_mfma_i32_32x32x32_i8.  Both operands are K-contiguous, so the
// MFMA "A" operand is a 32-row block of Wq (rows = output channels) and the "B"
// operand a 32-row block of Xq (rows = tokens); a lane then ends up holding four
// consecutive output channels of one token, which the epilogue writes as one
// 8-byte (bf16) or 16-byte (fp32/int32) store.  Tiles of Wq and Xq are staged
// through LDS in a double buffer (one barrier per K stage); the 16-byte chunk
// position within each LDS row is XOR-swizzled by the row index so that both the
// staging writes and the fragment reads (32 rows, same column) are free of bank
// conflicts.  Workgroups are remapped so that each XCD (which owns a private L2)
// works through a contiguous run of tiles, grouped 8 output-channel tiles wide,
// which keeps the operand panels it streams shared inside that L2.
#include "common.h"
#include "kernels.h"

namespace sq {

// Raw buffer resource over [base, base + bytes): loads whose VGPR offset is
// >= bytes return zero, which is how rows past the matrix edge become zero rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Four consecutive outputs of one row.  VEC: one 8/16-byte store (the caller
// guarantees all four exist: N % 4 == 0 and the first is in range); otherwise
// element stores of the nrem (>= 1) outputs that exist.
template <int OUT, bool VEC>
__device__ __forceinline__ void store4(void* Y, int64_t off, int nrem, const int* a, float sc_t,
                                       const float* wsv) {
  if (OUT == kOutI32) {
    int* y = static_cast<int*>(Y) + off;
    if (VEC) { *reinterpret_cast<int4*>(y) = make_int4(a[0], a[1], a[2], a[3]); return; }
    for (int e = 0; e < 4 && e < nrem; ++e) y[e] = a[e];
    return;
  }
  float v[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) v[e] = (float)a[e] * (sc_t * wsv[e]);
  if (OUT == kOutF32) {
    float* y = static_cast<float*>(Y) + off;
    if (VEC) { *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]); return; }
    for (int e = 0; e < 4 && e < nrem; ++e) y[e] = v[e];
  } else {
    uint16_t* y = static_cast<uint16_t*>(Y) + off;
    if (VEC) {
      uint2 p;
      p.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
      p.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
      *reinterpret_cast<uint2*>(y) = p;
      return;
    }
    for (int e = 0; e < 4 && e < nrem; ++e) y[e] = (uint16_t)f32_to_bf16(v[e]);
  }
}

// Tile order: XCD-contiguous runs, then groups of 8 output-channel tiles.
__device__ __forceinline__ void tile_coords(int bid, int G, int tiles_n, int tiles_t, int& tn, int& tt) {
  const int xcd = bid & 7, idx = bid >> 3;
  const int q = G >> 3, rem = G & 7;
  const int logical = xcd * q + (xcd < rem ? xcd : rem) + idx;
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_t;
  const int g = logical / per_group, within = logical - g * per_group;
  const int gn = tiles_n - g * GROUP < GROUP ? tiles_n - g * GROUP : GROUP;
  tn = g * GROUP + within % gn;
  tt = within / gn;
}

// Requires K % 16 == 0, (N + BN) * K < 2^31 and (T + BT) * K < 2^31 (the host
// splits larger problems), 16-byte aligned Xq and Wq.
template <int BN, int BT, int BK, int WN, int WT, int OUT, bool VEC>
__global__ __launch_bounds__(WN* WT * 64) void gemm_i8_mfma_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ xs, const int8_t* __restrict__ Wq,
    const float* __restrict__ ws, int T, int N, int K, void* __restrict__ Y, int64_t ldy,
    int tiles_n, int tiles_t) {
  constexpr int NT = WN * WT * 64;
  constexpr int CPR = BK / 16;                 // 16-byte chunks per LDS row
  constexpr int RPB = 16 / CPR;                // LDS rows per 256-byte bank line
  constexpr int RSTEP = NT / CPR;              // rows covered by one staging pass
  constexpr int WTN = BN / WN, WTT = BT / WT;  // wave tile
  constexpr int RN = WTN / 32, RT = WTT / 32;  // 32x32 MFMA blocks per wave
  constexpr int A_LD = BN / RSTEP, B_LD = BT / RSTEP;
  static_assert(A_LD * RSTEP == BN && B_LD * RSTEP == BT && RSTEP % 16 == 0, "tile/threads mismatch");
  __shared__ __attribute__((aligned(16))) int8_t lds[2][(BN + BT) * BK];

  int tn, tt;
  tile_coords(blockIdx.x, gridDim.x, tiles_n, tiles_t, tn, tt);
  const int n0 = tn * BN, t0 = tt * BT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wt = wave / WN;

  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(Wq, N * K);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(Xq, T * K);

  // staging: this thread moves chunk c of rows r0 + p*RSTEP (p < A_LD / B_LD)
  const int c = tid % CPR, r0 = tid / CPR;
  const int a_goff = (n0 + r0) * K + c * 16;
  const int b_goff = (t0 + r0) * K + c * 16;
  const int st_off = r0 * BK + ((c ^ ((r0 / RPB) % CPR)) * 16);   // same swizzle for every p

  // The whole byte offset goes in the VGPR operand: the buffer range check
  // covers that operand (not the scalar one), so rows past the edge and masked
  // K-tail chunks (sent to kOob) read as zero and never leave the allocation.
  constexpr int kOob = 0x7FFFFFF0;
  v4i ra[A_LD], rb[B_LD];
  auto gload = [&](int k0) {
    const bool kin = c * 16 < K - k0;   // false only in a partial last K stage
#pragma unroll
    for (int p = 0; p < A_LD; ++p)
      ra[p] = __builtin_amdgcn_raw_buffer_load_b128(rsA, kin ? a_goff + p * RSTEP * K + k0 : kOob, 0, 0);
#pragma unroll
    for (int p = 0; p < B_LD; ++p)
      rb[p] = __builtin_amdgcn_raw_buffer_load_b128(rsB, kin ? b_goff + p * RSTEP * K + k0 : kOob, 0, 0);
  };
  auto lstore = [&](int buf) {
    int8_t* base = &lds[buf][st_off];
#pragma unroll
    for (int p = 0; p < A_LD; ++p) *reinterpret_cast<v4i*>(base + p * RSTEP * BK) = ra[p];
#pragma unroll
    for (int p = 0; p < B_LD; ++p) *reinterpret_cast<v4i*>(base + BN * BK + p * RSTEP * BK) = rb[p];
  };

  // fragment reads: rows wn*WTN + i*32 + fr (A) and wt*WTT + j*32 + fr (B); the
  // block offsets are multiples of 16 rows, so the swizzle depends on fr only
  const int fr = lane & 31, fc = lane >> 5;
  const int sw = (fr / RPB) % CPR;
  const int a_base = (wn * WTN + fr) * BK;
  const int b_base = BN * BK + (wt * WTT + fr) * BK;
  int cofs[BK / 32];
#pragma unroll
  for (int kk = 0; kk < BK / 32; ++kk) cofs[kk] = ((kk * 2 + fc) ^ sw) * 16;

  v16i acc[RN][RT];
#pragma unroll
  for (int i = 0; i < RN; ++i)
#pragma unroll
    for (int j = 0; j < RT; ++j) acc[i][j] = v16i{};

  const int nst = (K + BK - 1) / BK;
  gload(0);
  lstore(0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const int cur = s & 1;
    if (s + 1 < nst) gload((s + 1) * BK);
    const int8_t* L = &lds[cur][0];
#pragma unroll
    for (int kk = 0; kk < BK / 32; ++kk) {
      v4i fa[RN], fb[RT];
#pragma unroll
      for (int i = 0; i < RN; ++i)
        fa[i] = *reinterpret_cast<const v4i*>(L + a_base + cofs[kk] + i * 32 * BK);
#pragma unroll
      for (int j = 0; j < RT; ++j)
        fb[j] = *reinterpret_cast<const v4i*>(L + b_base + cofs[kk] + j * 32 * BK);
#pragma unroll
      for (int i = 0; i < RN; ++i)
#pragma unroll
        for (int j = 0; j < RT; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[i], fb[j], acc[i][j], 0, 0, 0);
    }
    if (s + 1 < nst) lstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: per block (i, j) and group g the lane holds outputs
  // t = t0 + wt*WTT + j*32 + fr, n = n0 + wn*WTN + i*32 + 8g + 4*fc + 0..3
  float sc[RT];
  int tj[RT];
#pragma unroll
  for (int j = 0; j < RT; ++j) {
    tj[j] = t0 + wt * WTT + j * 32 + fr;
    sc[j] = (OUT != kOutI32 && tj[j] < T) ? xs[tj[j]] : 0.0f;
  }
#pragma unroll
  for (int i = 0; i < RN; ++i) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int n = n0 + wn * WTN + i * 32 + 8 * g + 4 * fc;
      if (n >= N) continue;
      float wsv[4] = {0.f, 0.f, 0.f, 0.f};
      if (OUT != kOutI32) {
        if (VEC) {
          const float4 w4 = *reinterpret_cast<const float4*>(ws + n);
          wsv[0] = w4.x; wsv[1] = w4.y; wsv[2] = w4.z; wsv[3] = w4.w;
        } else {
          for (int e = 0; e < 4; ++e) wsv[e] = (n + e < N) ? ws[n + e] : 0.0f;
        }
      }
#pragma unroll
      for (int j = 0; j < RT; ++j) {
        if (tj[j] >= T) continue;
        const int a4[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2],
                           acc[i][j][4 * g + 3]};
        store4<OUT, VEC>(Y, (int64_t)tj[j] * ldy + n, N - n, a4, sc[j], wsv);
      }
    }
  }
}

template <int BN, int BT, int BK, int WN, int WT, bool VEC>
static void launch_out(int out, dim3 grid, dim3 block, hipStream_t st, const int8_t* Xq, const float* xs,
                       const int8_t* Wq, const float* ws, int T, int N, int K, void* Y, int64_t ldy,
                       int tiles_n, int tiles_t) {
  switch (out) {
    case kOutF32:
      hipLaunchKernelGGL((gemm_i8_mfma_kernel<BN, BT, BK, WN, WT, kOutF32, VEC>), grid, block, 0, st, Xq, xs, Wq,
                         ws, T, N, K, Y, ldy, tiles_n, tiles_t);
      break;
    case kOutBF16:
      hipLaunchKernelGGL((gemm_i8_mfma_kernel<BN, BT, BK, WN, WT, kOutBF16, VEC>), grid, block, 0, st, Xq, xs, Wq,
                         ws, T, N, K, Y, ldy, tiles_n, tiles_t);
      break;
    default:
      hipLaunchKernelGGL((gemm_i8_mfma_kernel<BN, BT, BK, WN, WT, kOutI32, VEC>), grid, block, 0, st, Xq, xs, Wq,
                         ws, T, N, K, Y, ldy, tiles_n, tiles_t);
      break;
  }
}

template <int BN, int BT, int BK, int WN, int WT>
static hipError_t gemm_cfg(const GemmArgs& a, hipStream_t st) {
  // Split so that every operand slice handed to one launch spans < 2^31 bytes
  // (32-bit buffer offsets), counting one tile of overhang past the edge.
  const int64_t lim = (int64_t)1 << 31;
  const int64_t n_chunk = ((lim / a.K - BN) / BN) * BN;
  const int64_t t_chunk = ((lim / a.K - BT) / BT) * BT;
  const size_t osz = a.out == kOutBF16 ? 2 : 4;
  for (int64_t tb = 0; tb < a.T; tb += t_chunk) {
    const int T = (int)(a.T - tb < t_chunk ? a.T - tb : t_chunk);
    for (int64_t nb = 0; nb < a.N; nb += n_chunk) {
      const int N = (int)(a.N - nb < n_chunk ? a.N - nb : n_chunk);
      const int tiles_n = (N + BN - 1) / BN, tiles_t = (T + BT - 1) / BT;
      dim3 grid(tiles_n * tiles_t), block(WN * WT * 64);
      const int8_t* Xq = a.Xq + tb * a.K;
      const int8_t* Wq = a.Wq + nb * a.K;
      const float* xs = a.xs ? a.xs + tb : nullptr;
      const float* ws = a.ws ? a.ws + nb : nullptr;
      void* Y = static_cast<char*>(a.Y) + (tb * a.N + nb) * osz;
      // a column slice of Y keeps 16-byte alignment only if nb is a multiple of 4
      // a column slice of Y keeps 16-byte alignment only if nb is a multiple of 4
      const bool vs = a.vec_store && nb % 4 == 0;
      const int K = (int)a.K;
      if (vs) launch_out<BN, BT, BK, WN, WT, true>(a.out, grid, block, st, Xq, xs, Wq, ws, T, N, K, Y, a.N, tiles_n, tiles_t);
      else launch_out<BN, BT, BK, WN, WT, false>(a.out, grid, block, st, Xq, xs, Wq, ws, T, N, K, Y, a.N, tiles_n, tiles_t);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_gemm_mfma(const GemmArgs& a, int ncu, hipStream_t st) {
  // 256x256 tiles when they fill the chip at least once, else 128x128.
  const int64_t big = ((a.N + 255) / 256) * ((a.T + 255) / 256);
  if (big >= ncu) return gemm_cfg<256, 256, 64, 2, 2>(a, st);
  return gemm_cfg<128, 128, 64, 2, 2>(a, st);
}

// ---------------------------------------------------------------- generic path
template <int OUT>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const int8_t* __restrict__ Xq,
                                                           const float* __restrict__ xs,
                                                           const int8_t* __restrict__ Wq,
                                                           const float* __restrict__ ws, int64_t T,
                                                           int64_t N, int64_t K, void* __restrict__ Y) {
  const int64_t total = T * N;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = o / N, n = o - t * N;
    const int8_t* x = Xq + t * K;
    const int8_t* w = Wq + n * K;
    int acc = 0;
    for (int64_t k = 0; k < K; ++k) acc += (int)x[k] * (int)w[k];
    if (OUT == kOutI32) {
      static_cast<int*>(Y)[o] = acc;
    } else {
      const float v = (float)acc * (xs[t] * ws[n]);
      if (OUT == kOutF32) static_cast<float*>(Y)[o] = v;
      else static_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_bf16(v);
    }
  }
}

hipError_t launch_gemm_generic(const GemmArgs& a, hipStream_t st) {
  int64_t total = a.T * a.N;
  int64_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  dim3 grid((unsigned)g), block(256);
  switch (a.out) {
    case kOutF32:
      hipLaunchKernelGGL(gemm_generic_kernel<kOutF32>, grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y);
      break;
    case kOutBF16:
      hipLaunchKernelGGL(gemm_generic_kernel<kOutBF16>, grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y);
      break;
    default:
      hipLaunchKernelGGL(gemm_generic_kernel<kOutI32>, grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y);
      break;
  }
  return hipGetLastError();
}

}  // namespace sq
