// Decode-shaped W8A8 GEMM (few tokens, T <= 64) on gfx950.
//
// With a handful of tokens the layer is bound by streaming the int8 weights from
// HBM (multigrid.ai "SmoothQuant Explained", section "Where it fits, and where it
// does not": at small batch the multiply is not the bottleneck), so the kernel is
// built around reading Wq at the highest rate the memory system gives:
//   * each weight load instruction reads whole row segments (KC = 256 contiguous
//     bytes of each of 4 rows), non-temporal, since every weight byte is used once;
//   * the next chunk's loads are issued into a two-slot register ring before
//     the current chunk is processed; they sit under a branch (q + 1 < nit), so
//     the compiler waits for them too before the chunk's transpose completes,
//     and a wave has one chunk in flight that drains; a straight-line loop with
//     one to two chunks always in flight measured slower for int8 (42.0 ->
//     43.6 us on 16 x 28672 x 8192) and within a few per cent for FP8;
//   * a workgroup owns NB*16 output channels; its KW waves take alternate K
//     chunks (on layers that fill the CUs KW = 2 measured equal to or up to ~2%
//     faster than 1 depending on the GPU and 4 clearly slower; where each CU holds
//     a single workgroup 4 is faster), then add their int32 partial sums exactly through
//     LDS; each wave re-reads the small activation codes (L2-resident) once per
//     chunk for all of its channels;
//   * the epilogue's scale factors, and the decomposition's outlier operands
//     (copied into LDS), are fetched before the K loop, so no memory round trip
//     is left for the end of a workgroup.
// v_mfma_i32_16x16x64_i8 wants a 16-row block of Wq with lane l holding 16 bytes
// of row l%16, so each chunk is transposed through a per-wave LDS tile: rows are
// written as loaded and read back in the MFMA layout, with the 16-byte chunk
// position XOR-swizzled by row so that the 16 rows of one read hit distinct banks.
// The token codes are operand B (16 tokens per MFMA).  Integer accumulation is
// exact; the epilogue is y = fl32(fl32(acc) * fl32(x_scale[t] * w_scale[n])).
//
// A second form, gemv_seg_kernel, serves wide layers with deep K at up to 16
// tokens: each load instruction reads 1 KB of one weight row, see its comment.
#include <type_traits>
#include <utility>

#include "common.h"
#include "kernels.h"
#include "trace.h"
#include "slices.h"

namespace sq {

typedef float v4f __attribute__((ext_vector_type(4)));

namespace {

[[maybe_unused]] __device__ __forceinline__ __amdgpu_buffer_rsrc_t gemv_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// s_waitcnt immediate for "vmcnt <= n", other counters unconstrained (gfx9
// encoding: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
[[maybe_unused]] constexpr int seg_vmcnt(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }

template <int... I, typename F>
__device__ __forceinline__ void static_for(std::integer_sequence<int, I...>, F&& f) {
  (f(std::integral_constant<int, I>{}), ...);
}

}  // namespace

// so[i][b][e] = sum over o ascending of xo[o][t] * wo[o][n] for the lane's token
// t = b*16 + fi and channel n = n0 + i*16 + 4*fg + e, channel blocks I0 <= i < I1;
// one binary32 rounding per multiply and per add.  Each step reads the lane's
// token values and channel quadruples once (from the LDS copies ox [n_o][TB*16]
// and ow [n_o][NB*16] when staged, else from xo / wo) and advances all the sums.
// Entries past T or N are zero and never stored.
template <int NB, int TB, int I0, int I1>
__device__ __forceinline__ void gemv_outlier_sums(float (&so)[NB][TB][4], int n_o, int stage,
                                                  const float* ox, const float* ow, const float* __restrict__ xo,
                                                  int64_t ldxo, const float* __restrict__ wo, int64_t ldwo, int T,
                                                  int N, int n0, int fi, int fg) {
  constexpr int TL = TB * 16, CL = NB * 16;
  // operands of outlier o: token values xb[b], channel quadruples wi[i][e]
  auto fetch = [&](int o, float* xb, float (*wi)[4]) {
    if (stage) {
#pragma unroll
      for (int b = 0; b < TB; ++b) xb[b] = ox[o * TL + b * 16 + fi];
#pragma unroll
      for (int i = I0; i < I1; ++i) {
        const float4 w4 = *reinterpret_cast<const float4*>(ow + o * CL + i * 16 + 4 * fg);
        wi[i][0] = w4.x; wi[i][1] = w4.y; wi[i][2] = w4.z; wi[i][3] = w4.w;
      }
    } else {
#pragma unroll
      for (int b = 0; b < TB; ++b) xb[b] = b * 16 + fi < T ? xo[(int64_t)o * ldxo + b * 16 + fi] : 0.0f;
#pragma unroll
      for (int i = I0; i < I1; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int n = n0 + i * 16 + 4 * fg + e;
          wi[i][e] = n < N ? wo[(int64_t)o * ldwo + n] : 0.0f;
        }
    }
  };
  auto step = [&](const float* xb, const float (*wi)[4]) {
#pragma unroll
    for (int i = I0; i < I1; ++i)
#pragma unroll
      for (int b = 0; b < TB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e) so[i][b][e] = so[i][b][e] + xb[b] * wi[i][e];
  };
  // four outliers' operands are fetched before their four steps (in order)
  int o = 0;
  for (; o + 4 <= n_o; o += 4) {
    float xb[4][TB], wi[4][NB][4];
#pragma unroll
    for (int u = 0; u < 4; ++u) fetch(o + u, xb[u], wi[u]);
#pragma unroll
    for (int u = 0; u < 4; ++u) step(xb[u], wi[u]);
  }
  for (; o < n_o; ++o) {
    float xb[TB], wi[NB][4];
    fetch(o, xb, wi);
    step(xb, wi);
  }
}

// Requires K % 16 == 0, N * K < 2^31 and T * K < 2^31 (the host splits larger N),
// 16-byte aligned Xq and Wq.  KW waves per workgroup, which owns NB*16 channels.
// F8: the codes are FP8 E4M3 and each pair of 64-byte k-steps is one
// v_mfma_f32_16x16x128_f8f6f4 (binary32 accumulators; the scaled builtin with
// zero scale operands, for which the compiler selects the unscaled instruction,
// bit-identical on the GPU to E8M0 unit scales):
// a lane joins the two 16-byte chunks it would take for the two int8 steps, for
// the weights and the token codes alike, so every product pairs the same k.
// OUTL: the epilogue adds the binary32 outlier-channel product of the
// mixed-precision decomposition, sum over o ascending of xo[o][t] * wo[o][n].
template <int NB, int TB, int OUT, int KW, bool OUTL, bool F8>
__global__ __launch_bounds__(64 * KW) void gemv_i8_mfma_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ xs, const int8_t* __restrict__ Wq,
    const float* __restrict__ ws, int T, int N, int K, void* __restrict__ Y, int64_t ldy, int vec_store,
    const float* __restrict__ xo, int64_t ldxo, const float* __restrict__ wo, int64_t ldwo, int n_o,
    int stage) {
  // The body exists only in the device pass (the host pass needs just the stub).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int KC = 256;                 // K bytes per chunk
  constexpr int D = 2;                    // chunks in the register ring
  constexpr int CPRW = KC / 16;           // 16-byte pieces per row per chunk (16)
  constexpr int RPI = 64 / CPRW;          // rows per load instruction (4)
  constexpr int NI = 16 * NB / RPI;       // weight loads per chunk per lane
  constexpr int KS = KC / 64;             // MFMA k-steps per chunk (4)
  constexpr int kOob = 0x7FFFFFF0;        // offset the range check turns into zeros
  __shared__ __attribute__((aligned(1024))) int8_t lds_all[KW][16 * NB * KC];
  static_assert(KW * NB * TB * 64 * 16 <= KW * 16 * NB * KC, "partial and outlier sums must fit the LDS tiles");
  static_assert(!OUTL || KW <= 2, "the outlier sums are split between at most two waves");
  const int lane = threadIdx.x & 63, kw = threadIdx.x >> 6;
  int8_t* lds = lds_all[kw];   // this wave's transpose tile
  const int n0 = blockIdx.x * 16 * NB;
  const __amdgpu_buffer_rsrc_t rsW = gemv_rsrc(Wq, N * K);   // rows >= N read as zeros
  const __amdgpu_buffer_rsrc_t rsX = gemv_rsrc(Xq, T * K);   // tokens >= T read as zeros

  // weight loads: instruction p covers rows p*RPI .. +RPI-1, lane -> (row, piece)
  const int dr = lane / CPRW, dc = lane % CPRW;
  int w_off[NI], w_lds[NI];
#pragma unroll
  for (int p = 0; p < NI; ++p) {
    const int rr = p * RPI + dr;
    w_off[p] = (n0 + rr) * K + dc * 16;
    w_lds[p] = rr * KC + ((dc ^ (rr & 15)) * 16);
  }
  // operand reads: lane (fi = lane%16, fg = lane/16); k-step m uses piece m*4 + fg
  const int fi = lane & 15, fg = lane >> 4;
  int xoff[TB];
#pragma unroll
  for (int b = 0; b < TB; ++b) xoff[b] = (b * 16 + fi) * K + fg * 16;

  // The epilogue's scale factors are fetched before the K loop: loaded after it,
  // they would add one more memory round trip to the end of every workgroup.
  float xsv[TB], wsv[NB][4];
#pragma unroll
  for (int b = 0; b < TB; ++b) xsv[b] = 0.0f;
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) wsv[i][e] = 0.0f;
  if (OUT != kOutI32 && kw == 0) {
#pragma unroll
    for (int b = 0; b < TB; ++b)
      if (b * 16 + fi < T) xsv[b] = xs[b * 16 + fi];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n0 + i * 16 + 4 * fg + e < N) wsv[i][e] = ws[n0 + i * 16 + 4 * fg + e];
  }

  static_assert(!(F8 && (OUTL || OUT == kOutI32)), "FP8: float outputs, no outlier term");
  using AccT = std::conditional_t<F8, v4f, v4i>;
  AccT acc[NB][TB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int b = 0; b < TB; ++b) acc[i][b] = AccT{0, 0, 0, 0};

  v4i wr[D][NI], xv[D][TB][KS];
  auto load = [&](auto slot_c, int k0) {
    constexpr int sl = decltype(slot_c)::value;
    const bool kin = dc * 16 < K - k0;
#pragma unroll
    for (int p = 0; p < NI; ++p)   // cache policy 2: non-temporal
      wr[sl][p] = __builtin_amdgcn_raw_buffer_load_b128(rsW, kin ? w_off[p] + k0 : kOob, 0, 2);
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int m = 0; m < KS; ++m)
        xv[sl][b][m] = __builtin_amdgcn_raw_buffer_load_b128(
            rsX, (k0 + m * 64 + fg * 16 < K) ? xoff[b] + k0 + m * 64 : kOob, 0, 0);
  };
  auto compute = [&](auto slot_c) {
    constexpr int sl = decltype(slot_c)::value;
#pragma unroll
    for (int p = 0; p < NI; ++p) *reinterpret_cast<v4i*>(lds + w_lds[p]) = wr[sl][p];
    if constexpr (F8) {
#pragma unroll
      for (int m = 0; m < KS; m += 2) {
        const int c0 = m * 4 + fg, c1 = c0 + 4;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const v8i wv = __builtin_shufflevector(
              *reinterpret_cast<const v4i*>(lds + (i * 16 + fi) * KC + ((c0 ^ fi) * 16)),
              *reinterpret_cast<const v4i*>(lds + (i * 16 + fi) * KC + ((c1 ^ fi) * 16)), 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            const v8i x8 = __builtin_shufflevector(xv[sl][b][m], xv[sl][b][m + 1], 0, 1, 2, 3, 4, 5, 6, 7);
            acc[i][b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, x8, acc[i][b], 0, 0, 0, 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int m = 0; m < KS; ++m) {
        const int c = m * 4 + fg;
#pragma unroll
        for (int i = 0; i < NB; ++i) {
          const v4i wv = *reinterpret_cast<const v4i*>(lds + (i * 16 + fi) * KC + ((c ^ fi) * 16));
#pragma unroll
          for (int b = 0; b < TB; ++b)
            acc[i][b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(wv, xv[sl][b][m], acc[i][b], 0, 0, 0);
        }
      }
    }
  };

  // this wave's chunks: kw, kw + KW, kw + 2 KW, ...
  const int nall = (K + KC - 1) / KC;
  const int nit = nall > kw ? (nall - kw + KW - 1) / KW : 0;
  // Outlier operands of this workgroup's outputs (stage != 0): the token values
  // xo[o][t < TB*16] and the channel values wo[o][n0 .. n0 + 16 NB) are copied into
  // LDS, 32 independent loads per thread at a time, so the epilogue reads them
  // from LDS.  The first batch is loaded before the first weight chunk is issued
  // and stored after it, so that its round trip overlaps the chunk's.
  constexpr int TL = TB * 16, CL = NB * 16;
  extern __shared__ __attribute__((aligned(16))) float gemv_outl[];
  float* ox = gemv_outl;             // [n_o][TL]
  float* ow = gemv_outl + n_o * TL;  // [n_o][CL]
  const int nx = n_o * TL, ntot = nx + n_o * CL;
  auto stage_load = [&](int q) {
    float v = 0.0f;
    if (q < nx) {
      const int o = q / TL, tl = q - o * TL;
      if (tl < T) v = xo[(int64_t)o * ldxo + tl];
    } else if (q < ntot) {
      const int o = (q - nx) / CL, c = q - nx - o * CL;
      if (n0 + c < N) v = wo[(int64_t)o * ldwo + n0 + c];
    }
    return v;
  };
  constexpr int SB = 32, SSTEP = SB * 64 * KW;   // loads per thread per batch, entries per batch
  float sv[SB];
  if (OUTL && stage) {
#pragma unroll
    for (int u = 0; u < SB; ++u) sv[u] = stage_load(threadIdx.x + u * 64 * KW);
  }

  static_for(std::make_integer_sequence<int, D - 1>{}, [&](auto u) {
    if (decltype(u)::value < nit) load(u, (decltype(u)::value * KW + kw) * KC);
  });

  if (OUTL && stage) {
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int q = threadIdx.x + u * 64 * KW;
      if (q < ntot) gemv_outl[q] = sv[u];
    }
    for (int q0 = threadIdx.x + SSTEP; q0 < ntot; q0 += SSTEP) {
#pragma unroll
      for (int u = 0; u < SB; ++u) sv[u] = stage_load(q0 + u * 64 * KW);
#pragma unroll
      for (int u = 0; u < SB; ++u) {
        const int q = q0 + u * 64 * KW;
        if (q < ntot) gemv_outl[q] = sv[u];
      }
    }
  }

  for (int q0 = 0; q0 < nit; q0 += D) {
    static_for(std::make_integer_sequence<int, D>{}, [&](auto u) {
      constexpr int uu = decltype(u)::value;
      const int q = q0 + uu;
      if (q + D - 1 < nit) load(std::integral_constant<int, (uu + D - 1) % D>{}, ((q + D - 1) * KW + kw) * KC);
      if (q < nit) compute(u);
    });
  }
  // Outlier-channel products of this lane's outputs (gemv_outlier_sums).  With
  // two waves, wave 0 forms the sums of channel blocks i < NB/2 and wave 1 those
  // of the others, at the same time; each sum is formed by one wave.
  float so[NB][TB][4];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) so[i][b][e] = 0.0f;
  auto outlier_sums = [&]() {
    if (KW == 1)
      gemv_outlier_sums<NB, TB, 0, NB>(so, n_o, stage, ox, ow, xo, ldxo, wo, ldwo, T, N, n0, fi, fg);
    else if (kw == 0)
      gemv_outlier_sums<NB, TB, 0, NB / 2>(so, n_o, stage, ox, ow, xo, ldxo, wo, ldwo, T, N, n0, fi, fg);
    else
      gemv_outlier_sums<NB, TB, NB / 2, NB>(so, n_o, stage, ox, ow, xo, ldxo, wo, ldwo, T, N, n0, fi, fg);
  };

  if (KW > 1) {
    // exact integer sum of the KW partial accumulators; the LDS tiles are free
    // once every wave has passed the first barrier
    __syncthreads();
    AccT* red = reinterpret_cast<AccT*>(&lds_all[0][0]);
    float4* sor = reinterpret_cast<float4*>(red + (KW - 1) * NB * TB * 64);
    if (kw > 0) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int b = 0; b < TB; ++b) red[((kw - 1) * NB * TB + i * TB + b) * 64 + lane] = acc[i][b];
    }
    if (OUTL) {
      outlier_sums();
      if (kw == 1) {
#pragma unroll
        for (int i = NB / 2; i < NB; ++i)
#pragma unroll
          for (int b = 0; b < TB; ++b)
            sor[(i * TB + b) * 64 + lane] = make_float4(so[i][b][0], so[i][b][1], so[i][b][2], so[i][b][3]);
      }
    }
    __syncthreads();
    if (kw > 0) return;
#pragma unroll
    for (int w = 1; w < KW; ++w)
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int b = 0; b < TB; ++b) acc[i][b] += red[((w - 1) * NB * TB + i * TB + b) * 64 + lane];
    if (OUTL) {
#pragma unroll
      for (int i = NB / 2; i < NB; ++i)
#pragma unroll
        for (int b = 0; b < TB; ++b) {
          const float4 f = sor[(i * TB + b) * 64 + lane];
          so[i][b][0] = f.x; so[i][b][1] = f.y; so[i][b][2] = f.z; so[i][b][3] = f.w;
        }
    }
  } else if (OUTL) {
    if (stage) __syncthreads();
    outlier_sums();
  }

  // epilogue: lane holds n = n0 + i*16 + 4*fg + 0..3 for token t = b*16 + fi
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int t = b * 16 + fi, n = n0 + i * 16 + 4 * fg;
      if (t >= T || n >= N) continue;
      const int nrem = N - n;
      const bool vec = vec_store && nrem >= 4;
      const AccT a4 = acc[i][b];
      if (OUT == kOutI32) {
        int* y = static_cast<int*>(Y) + (int64_t)t * ldy + n;
        if (vec) *reinterpret_cast<int4*>(y) = make_int4(a4[0], a4[1], a4[2], a4[3]);
        else for (int e = 0; e < 4 && e < nrem; ++e) y[e] = a4[e];
        continue;
      }
      const float sc = xsv[b];
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = (e < nrem) ? (float)a4[e] * (sc * wsv[i][e]) : 0.0f;
      if (OUTL) {
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = v[e] + so[i][b][e];
      }
      if (OUT == kOutF32) {
        float* y = static_cast<float*>(Y) + (int64_t)t * ldy + n;
        if (vec) *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
        else for (int e = 0; e < 4 && e < nrem; ++e) y[e] = v[e];
      } else {
        uint16_t* y = static_cast<uint16_t*>(Y) + (int64_t)t * ldy + n;
        if (vec) {
          uint2 pk;
          pk.x = f32x2_to_bf16x2(v[0], v[1]);
          pk.y = f32x2_to_bf16x2(v[2], v[3]);
          *reinterpret_cast<uint2*>(y) = pk;
        } else {
          for (int e = 0; e < 4 && e < nrem; ++e) y[e] = (uint16_t)f32_to_bf16(v[e]);
        }
      }
    }
#endif
}

// Decode form for wide layers with deep K, up to 16 tokens.  Every weight load
// instruction reads 1 KB of one row (64 lanes x 16 bytes), so a wave's reads are
// whole kilobyte runs of the rows.  The time of such reads did not depend on
// where the weight pages landed, unlike the 256-byte row pieces of
// gemv_i8_mfma_kernel (16 x 28672 x 8192: this form 39.8-40.3 us on each of three
// fresh allocations in one run, the other 37.8-45.8 us over several).  A workgroup owns
// 64 channels (four 16-channel blocks) and four waves, which take alternate 1 KB
// segments of K.  For one segment a wave keeps the 16 tokens' codes in
// registers and streams its four channel blocks through a single register slot.
// A block's 16 loaded rows are written to the wave's LDS tile, whose row pitch
// is 1040 bytes so that an MFMA read of 16 rows hits distinct banks, in two
// halves: each half as soon as it has landed, its registers then reloaded at
// once with the same half of the next block.  Then the block's 16 k-steps run
// from LDS.  So 8 to 16 rows per wave (8-16 KB) are always in flight; waiting
// for all 16 rows before reloading any measured 5% slower (41.8-42.0 against
// 39.8-40.0 us on 16 x 28672 x 8192).  The partial sums of the four waves are
// added exactly (int32) or in wave order (FP8, binary32) through LDS; the
// epilogue is that of gemv_i8_mfma_kernel.  Requires T <= 16, K % 16 == 0,
// (N + 64) * K <= 2^31 and T * K < 2^31 (the host slices N), and 16-byte aligned
// Xq and Wq.
// OUTL: the epilogue adds the decomposition's outlier-channel product (as in
// gemv_i8_mfma_kernel, same order and roundings).  The workgroup's operands,
// xo[o][t < 16] and wo[o][n0 .. n0 + 64), are copied into dynamic LDS before
// the K loop, at most kSegOutlierLoads loads per thread, so the host sends at
// most kSegMaxOutliers outliers here; each wave forms the sums of one channel
// block after the K loop.
constexpr int kSegOutlierLoads = 16;
constexpr int kSegMaxOutliers = 48;   // 48 x 320 B + 66.5 KB: two workgroups per CU
static_assert(kSegMaxOutliers * (16 + 64) <= kSegOutlierLoads * 256, "one batch of staging loads");
template <int OUT, bool OUTL, bool F8>
__global__ __launch_bounds__(256) void gemv_seg_kernel(const int8_t* __restrict__ Xq, const float* __restrict__ xs,
                                                       const int8_t* __restrict__ Wq, const float* __restrict__ ws,
                                                       int T, int N, int K, void* __restrict__ Y, int64_t ldy,
                                                       int vec_store, const float* __restrict__ xo, int64_t ldxo,
                                                       const float* __restrict__ wo, int64_t ldwo, int n_o) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NB = 4, KW = 4;           // channel blocks per workgroup, K-split waves
  constexpr int SEG = 1024;               // K bytes per segment
  constexpr int ROWB = SEG + 16;          // LDS row pitch
  constexpr int TILE = 16 * ROWB;         // one wave's tile: 16 rows of a segment
  constexpr int KS = SEG / 64;            // MFMA k-steps per segment (16)
  constexpr int kOob = 0x7FFFFFF0;        // offset the range check turns into zeros
  __shared__ __attribute__((aligned(16))) int8_t lds_all[KW * TILE];
  static_assert((KW - 1) * NB * 64 * 16 + (KW - 1) * 64 * 16 <= KW * TILE,
                "partial and outlier sums must fit the LDS tiles");
  static_assert(!(F8 && (OUTL || OUT == kOutI32)), "FP8: float outputs, no outlier term");
  const int lane = threadIdx.x & 63, kw = threadIdx.x >> 6;
  int8_t* tile = lds_all + kw * TILE;
  const int n0 = blockIdx.x * 16 * NB;
  const __amdgpu_buffer_rsrc_t rsW = gemv_rsrc(Wq, N * K);   // rows >= N read as zeros
  const __amdgpu_buffer_rsrc_t rsX = gemv_rsrc(Xq, T * K);   // tokens >= T read as zeros
  const int fi = lane & 15, fg = lane >> 4;
  // this wave's segments: kw, kw + KW, ...; unit u = (segment u / NB, block u % NB)
  const int nall = (K + SEG - 1) / SEG;
  const int nseg = nall > kw ? (nall - kw + KW - 1) / KW : 0;
  const int U = nseg * NB;

  // epilogue scale factors, fetched before the K loop (see gemv_i8_mfma_kernel)
  float xsv = 0.0f, wsv[NB][4];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) wsv[i][e] = 0.0f;
  if (OUT != kOutI32 && kw == 0) {
    if (fi < T) xsv = xs[fi];
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (n0 + i * 16 + 4 * fg + e < N) wsv[i][e] = ws[n0 + i * 16 + 4 * fg + e];
  }

  // rows n0 + 16 b .. +15 of unit u's segment: row r is one instruction, lane ->
  // bytes lane*16 .. +15 of the segment (cache policy 2: non-temporal)
  v4i wr[16];
  auto load_rows_at = [&](int u, int r0, int r1) {
    const int j = u / NB, b = u - j * NB;
    const int k0 = (j * KW + kw) * SEG + lane * 16;
    const bool in = u < U && k0 < K;
#pragma unroll
    for (int r = r0; r < r1; ++r)
      wr[r] = __builtin_amdgcn_raw_buffer_load_b128(rsW, in ? (n0 + b * 16 + r) * K + k0 : kOob, 0, 2);
  };
  auto load_rows = [&](int u) { load_rows_at(u, 0, 16); };
  // token codes of segment j in operand-B layout: token fi, k-step m, piece fg
  v4i tok[KS];
  auto load_tokens = [&](int j) {
    const int kb = (j * KW + kw) * SEG + fg * 16;
    const bool in = j < nseg;
#pragma unroll
    for (int m = 0; m < KS; ++m) {
      const int k = kb + m * 64;
      tok[m] = __builtin_amdgcn_raw_buffer_load_b128(rsX, (in && k < K) ? fi * K + k : kOob, 0, 0);
    }
  };

  using AccT = std::conditional_t<F8, v4f, v4i>;
  AccT acc[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) acc[i] = AccT{0, 0, 0, 0};

  // The rows of a unit are taken in two halves: as soon as a half has landed it
  // is written to the tile and its registers are reloaded with the same half of
  // the next unit, so 8 to 16 rows per wave stay in flight.  Loads complete in
  // issue order for vmcnt; the counts below are the loads issued after the
  // awaited ones.
  auto unit = [&](auto b_c, int u) {
    constexpr int b = decltype(b_c)::value;
    // rows 0-7: after them come rows 8-15 and, for a segment's first block, the
    // segment's 16 token loads
    __builtin_amdgcn_s_waitcnt(b == 0 ? seg_vmcnt(8 + KS) : seg_vmcnt(8));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < 8; ++r) *reinterpret_cast<v4i*>(tile + r * ROWB + lane * 16) = wr[r];
    __builtin_amdgcn_sched_barrier(0);
    load_rows_at(u + 1, 0, 8);
    __builtin_amdgcn_sched_barrier(0);
    // rows 8-15 and the tokens: after them come the 8 loads just issued
    __builtin_amdgcn_s_waitcnt(seg_vmcnt(8));
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 8; r < 16; ++r) *reinterpret_cast<v4i*>(tile + r * ROWB + lane * 16) = wr[r];
    __builtin_amdgcn_sched_barrier(0);
    load_rows_at(u + 1, 8, 16);
    __builtin_amdgcn_sched_barrier(0);
    const int8_t* L = tile + fi * ROWB + fg * 16;
    if constexpr (F8) {
      // the two 16-byte pieces of k-steps m and m + 1, for weights and tokens alike
#pragma unroll
      for (int m = 0; m < KS; m += 2) {
        const v8i wv = __builtin_shufflevector(*reinterpret_cast<const v4i*>(L + m * 64),
                                               *reinterpret_cast<const v4i*>(L + (m + 1) * 64), 0, 1, 2, 3, 4, 5,
                                               6, 7);
        const v8i x8 = __builtin_shufflevector(tok[m], tok[m + 1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[b] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wv, x8, acc[b], 0, 0, 0, 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int m = 0; m < KS; ++m)
        acc[b] = __builtin_amdgcn_mfma_i32_16x16x64_i8(*reinterpret_cast<const v4i*>(L + m * 64), tok[m], acc[b],
                                                       0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (b == NB - 1) load_tokens(u / NB + 1);   // after the segment's last block
    __builtin_amdgcn_sched_barrier(0);
  };

  // outlier operands: entries [0, nx) are ox[o][t], then ow[o][c]
  constexpr int TL = 16, CL = 16 * NB;
  extern __shared__ __attribute__((aligned(16))) float seg_outl[];
  float* ox = seg_outl;
  float* ow = seg_outl + n_o * TL;
  const int nx = n_o * TL, ntot = nx + n_o * CL;
  float sv[kSegOutlierLoads];
  if constexpr (OUTL) {
#pragma unroll
    for (int u = 0; u < kSegOutlierLoads; ++u) {
      const int q = threadIdx.x + u * 256;
      float v = 0.0f;
      if (q < nx) {
        const int o = q / TL, tl = q - o * TL;
        if (tl < T) v = xo[(int64_t)o * ldxo + tl];
      } else if (q < ntot) {
        const int o = (q - nx) / CL, c = q - nx - o * CL;
        if (n0 + c < N) v = wo[(int64_t)o * ldwo + n0 + c];
      }
      sv[u] = v;
    }
  }
  load_rows(0);
  load_tokens(0);
  if constexpr (OUTL) {   // stored while the first rows are in flight
#pragma unroll
    for (int u = 0; u < kSegOutlierLoads; ++u) {
      const int q = threadIdx.x + u * 256;
      if (q < ntot) seg_outl[q] = sv[u];
    }
  }
  for (int u = 0; u < U; u += NB)
    static_for(std::make_integer_sequence<int, NB>{}, [&](auto b) { unit(b, u + decltype(b)::value); });
  // the loads issued past the last unit read zeros; let them land before the
  // LDS tiles are reused (the barrier also publishes the staged outlier operands)
  __builtin_amdgcn_s_waitcnt(seg_vmcnt(0));
  __syncthreads();
  AccT* red = reinterpret_cast<AccT*>(lds_all);
  float4* sor = reinterpret_cast<float4*>(red + (KW - 1) * NB * 64);
  if (kw > 0) {
#pragma unroll
    for (int i = 0; i < NB; ++i) red[((kw - 1) * NB + i) * 64 + lane] = acc[i];
  }
  // outlier-channel sums (gemv_outlier_sums): wave kw forms those of block kw
  float so[NB][1][4];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) so[i][0][e] = 0.0f;
  if constexpr (OUTL) {
    static_for(std::make_integer_sequence<int, NB>{}, [&](auto ic) {
      constexpr int i = decltype(ic)::value;
      if (kw == i) {
        gemv_outlier_sums<NB, 1, i, i + 1>(so, n_o, 1, ox, ow, xo, ldxo, wo, ldwo, T, N, n0, fi, fg);
        if (i > 0) sor[(i - 1) * 64 + lane] = make_float4(so[i][0][0], so[i][0][1], so[i][0][2], so[i][0][3]);
      }
    });
  }
  __syncthreads();
  if (kw > 0) return;
#pragma unroll
  for (int w = 1; w < KW; ++w)
#pragma unroll
    for (int i = 0; i < NB; ++i) acc[i] += red[((w - 1) * NB + i) * 64 + lane];
  if constexpr (OUTL) {
#pragma unroll
    for (int i = 1; i < NB; ++i) {
      const float4 f = sor[(i - 1) * 64 + lane];
      so[i][0][0] = f.x; so[i][0][1] = f.y; so[i][0][2] = f.z; so[i][0][3] = f.w;
    }
  }

  // epilogue: lane holds n = n0 + i*16 + 4*fg + 0..3 for token t = fi
  const int t = fi;
  if (t >= T) return;
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int n = n0 + i * 16 + 4 * fg;
    if (n >= N) continue;
    const int nrem = N - n;
    const bool vec = vec_store && nrem >= 4;
    const AccT a4 = acc[i];
    if (OUT == kOutI32) {
      int* y = static_cast<int*>(Y) + (int64_t)t * ldy + n;
      if (vec) *reinterpret_cast<int4*>(y) = make_int4(a4[0], a4[1], a4[2], a4[3]);
      else for (int e = 0; e < 4 && e < nrem; ++e) y[e] = a4[e];
      continue;
    }
    float v[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) v[e] = (e < nrem) ? (float)a4[e] * (xsv * wsv[i][e]) : 0.0f;
    if (OUTL) {
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = v[e] + so[i][0][e];
    }
    if (OUT == kOutF32) {
      float* y = static_cast<float*>(Y) + (int64_t)t * ldy + n;
      if (vec) *reinterpret_cast<float4*>(y) = make_float4(v[0], v[1], v[2], v[3]);
      else for (int e = 0; e < 4 && e < nrem; ++e) y[e] = v[e];
    } else {
      uint16_t* y = static_cast<uint16_t*>(Y) + (int64_t)t * ldy + n;
      if (vec) {
        uint2 pk;
        pk.x = f32x2_to_bf16x2(v[0], v[1]);
        pk.y = f32x2_to_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(y) = pk;
      } else {
        for (int e = 0; e < 4 && e < nrem; ++e) y[e] = (uint16_t)f32_to_bf16(v[e]);
      }
    }
  }
#endif
}

template <bool F8>
static hipError_t gemv_seg_cfg(const GemmArgs& a, hipStream_t st) {
  // split N so that one launch's weight slice spans < 2^31 bytes (32-bit offsets)
  const int64_t n_chunk = rows_per_slice(a.K, 64);
  const size_t osz = a.out == kOutBF16 ? 2 : 4;
  for (int64_t nb = 0; nb < a.N; nb += n_chunk) {
    const int N = (int)(a.N - nb < n_chunk ? a.N - nb : n_chunk);
    dim3 grid((N + 63) / 64), block(256);
    const int8_t* Wq = a.Wq + nb * a.K;
    const float* ws = a.ws ? a.ws + nb : nullptr;
    void* Y = static_cast<char*>(a.Y) + nb * osz;
    const int vs = (a.vec_store && nb % 4 == 0) ? 1 : 0;
    const int T = (int)a.T, K = (int)a.K;
    const bool outl = a.n_o > 0 && a.out != kOutI32;
    if (outl && (F8 || a.n_o > kSegMaxOutliers)) return hipErrorInvalidValue;
    const float* wo = outl ? a.wo + nb : nullptr;
    const int n_o = outl ? (int)a.n_o : 0;
    const size_t shm = (size_t)n_o * (16 + 64) * sizeof(float);
    SQ_TRACE("gemv_seg_i8_mfma 64 channels per workgroup, 4 k-split waves over 1 KB segments, out %s%s%s, "
             "T %d N %d K %d, grid %u x %u threads",
             a.out == kOutF32 ? "f32" : a.out == kOutBF16 ? "bf16" : "i32", outl ? ", outlier term (LDS)" : "",
             F8 ? ", fp8" : "", T, N, K, grid.x, block.x);
#define SQ_SEG_LAUNCH(O, L)                                                                                   \
  hipLaunchKernelGGL((gemv_seg_kernel<O, L, F8>), grid, block, shm, st, a.Xq, a.xs, Wq, ws, T, N, K, Y, a.N, vs, \
                     a.xo, a.T, wo, a.N, n_o)
    if constexpr (F8) {   // float outputs only (the ABI rejects int32 for FP8)
      if (a.out == kOutF32) SQ_SEG_LAUNCH(kOutF32, false); else SQ_SEG_LAUNCH(kOutBF16, false);
    } else {
      if (a.out == kOutF32) { if (outl) SQ_SEG_LAUNCH(kOutF32, true); else SQ_SEG_LAUNCH(kOutF32, false); }
      else if (a.out == kOutBF16) { if (outl) SQ_SEG_LAUNCH(kOutBF16, true); else SQ_SEG_LAUNCH(kOutBF16, false); }
      else SQ_SEG_LAUNCH(kOutI32, false);
    }
#undef SQ_SEG_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

constexpr size_t kGemvOutlierLds = 64 * 1024;

template <int NB, int TB, int KW, bool F8>
static hipError_t gemv_cfg(const GemmArgs& a, hipStream_t st) {
  // split N so that one launch's weight slice spans < 2^31 bytes (32-bit offsets)
  const int64_t n_chunk = rows_per_slice(a.K, 16 * NB);
  const size_t osz = a.out == kOutBF16 ? 2 : 4;
  for (int64_t nb = 0; nb < a.N; nb += n_chunk) {
    const int N = (int)(a.N - nb < n_chunk ? a.N - nb : n_chunk);
    dim3 grid((N + 16 * NB - 1) / (16 * NB)), block(64 * KW);
    const int8_t* Wq = a.Wq + nb * a.K;
    const float* ws = a.ws ? a.ws + nb : nullptr;
    void* Y = static_cast<char*>(a.Y) + nb * osz;
    const int vs = (a.vec_store && nb % 4 == 0) ? 1 : 0;
    const int T = (int)a.T, K = (int)a.K;
    const bool outl = a.n_o > 0 && a.out != kOutI32;
    const float* wo = outl ? a.wo + nb : nullptr;
    const int n_o = outl ? (int)a.n_o : 0;
    // outlier operands staged in LDS up to 64 KB per workgroup
    const size_t dyn = (size_t)n_o * 16 * (TB + NB) * sizeof(float);
    const int stage = (outl && dyn <= kGemvOutlierLds) ? 1 : 0;
    const size_t shm = stage ? dyn : 0;
    SQ_TRACE("gemv_i8_mfma %d channels x %d tokens per workgroup, %d k-split waves, out %s%s%s, T %d N %d K %d, "
             "grid %u x %u threads",
             16 * NB, 16 * TB, KW, a.out == kOutF32 ? "f32" : a.out == kOutBF16 ? "bf16" : "i32",
             outl ? (stage ? ", outlier term (LDS)" : ", outlier term") : "", F8 ? ", fp8" : "", T, N, K, grid.x,
             block.x);
#define SQ_GEMV_LAUNCH(O, L)                                                                             \
  hipLaunchKernelGGL((gemv_i8_mfma_kernel<NB, TB, O, KW, L, F8>), grid, block, shm, st, a.Xq, a.xs, Wq, ws, T, N, \
                     K, Y, a.N, vs, a.xo, a.T, wo, a.N, n_o, stage)
    if constexpr (F8) {   // float outputs only (the ABI rejects int32 for FP8)
      if (a.out == kOutF32) SQ_GEMV_LAUNCH(kOutF32, false); else SQ_GEMV_LAUNCH(kOutBF16, false);
    } else {
      switch (a.out) {
        case kOutF32:
          if constexpr (KW <= 2) { if (outl) SQ_GEMV_LAUNCH(kOutF32, true); else SQ_GEMV_LAUNCH(kOutF32, false); }
          else { if (outl) return hipErrorInvalidValue; SQ_GEMV_LAUNCH(kOutF32, false); }
          break;
        case kOutBF16:
          if constexpr (KW <= 2) { if (outl) SQ_GEMV_LAUNCH(kOutBF16, true); else SQ_GEMV_LAUNCH(kOutBF16, false); }
          else { if (outl) return hipErrorInvalidValue; SQ_GEMV_LAUNCH(kOutBF16, false); }
          break;
        default:
          SQ_GEMV_LAUNCH(kOutI32, false);
          break;
      }
    }
#undef SQ_GEMV_LAUNCH
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int NB, int KW, bool F8>
static hipError_t gemv_tokens(const GemmArgs& a, hipStream_t st) {
  if (a.T <= 16) return gemv_cfg<NB, 1, KW, F8>(a, st);
  if (a.T <= 32) return gemv_cfg<NB, 2, KW, F8>(a, st);
  return gemv_cfg<NB, 4, KW, F8>(a, st);
}

hipError_t launch_gemv_mfma(const GemmArgs& a, int ncu, hipStream_t st) {
  // Channels per workgroup (16 NB) and K-split waves (KW), by layer width; all
  // choices give identical int8 results (exact integer partial sums); for FP8 the
  // number of waves sets the order in which binary32 partial sums are added, so
  // different wave counts differ in the last bits, within the same error bound.
  // Layers of 3/4 of a 64-channel block per CU or more: 64 channels, 2 waves (with
  // 32 channels the register ring holds each chunk's token codes for every
  // 16-token block, and 17-64 tokens ran 16-29% slower: 28672 x 8192 54.7
  // against 45.1 us at 32 tokens; the larger ring fits in the AGPRs at one wave
  // per SIMD).  Narrower layers spread their channels over the CUs instead:
  // 16 channels per workgroup while that leaves at least one workgroup per CU
  // and the token codes re-read per workgroup stay small, else 32.  Measured
  // with the weights streamed from HBM, against 64 channels and 2 waves:
  // 4096 x 8192 at 16 tokens 9.9 against 17.6 us (16 channels, 4 waves), 8192 x
  // 8192 14.9 against 19.2 us (16 channels), 8192 x 28672 at 64 tokens 73.5
  // against 95.3 us (32 channels), 6144 x 4096 at 64 tokens 14.3 against 19.9 us.
  const bool outl = a.n_o > 0 && a.out != kOutI32;
  const int64_t c64 = (a.N + 63) / 64, c32 = (a.N + 31) / 32;
  // At least one 64-channel block per CU, up to 16 tokens, K a multiple of 4096
  // from 8192 up: the 1 KB-segment form (gemv_seg_kernel), whose four waves then
  // take equal shares of K.  Measured over one allocation of the weights each,
  // against the form below: 16384 x 8192 26.4 against 28.2 us, 28672 x 8192 41.8
  // against 43.5 (1 token 39.9 against 42.7), 24576 x 12288 55.8 against 60.9,
  // 49152 x 12288 94.2 against 126.8, 16384 x 16384 at 8 tokens 47.5 against
  // 62.2, 57344 x 8192 at 1 token 75.8 against 86.5.  It lost where the waves'
  // shares differ (16384 x 9216 29.5 against 26.3 us, 16384 x 14336 41.6 against
  // 39.5) and where each wave has a single segment, leaving nothing to overlap
  // (16384 x 5120 20.5 against 15.9).  With the decomposition's outlier term up
  // to kSegMaxOutliers outliers (operands staged in LDS at two workgroups per CU).
  if (a.T <= 16 && c64 >= ncu && a.K >= 8192 && a.K % 4096 == 0 &&
      (!outl || (!a.f8 && a.n_o <= kSegMaxOutliers)))
    return a.f8 ? gemv_seg_cfg<true>(a, st) : gemv_seg_cfg<false>(a, st);
  // Layers of 3/4 to one 64-channel block per CU, K >= 8192, up to 16 tokens:
  // 8 waves (12288 x 12288 at 1/16 tokens 27.6/30.0 against 32.2/33.7 us,
  // 12288 x 49152 94.4/103.2 against 105.3/112.3; at 28672 channels 8 waves lost)
  if (4 * c64 >= 3 * (int64_t)ncu && c64 < ncu && a.K >= 8192 && a.T <= 16 && !outl)
    return a.f8 ? gemv_cfg<4, 1, 8, true>(a, st) : gemv_cfg<4, 1, 8, false>(a, st);
  // 32-channel workgroups above 16 tokens only where they make at most one round
  // on the CUs: 10240 x 8192 at 32 tokens 29.3 us with 320 of them, 26.7 with
  // 160 of 64 channels
  if (4 * c64 >= 3 * (int64_t)ncu || (c32 > ncu && a.T > 16))
    return a.f8 ? gemv_tokens<4, 2, true>(a, st) : gemv_tokens<4, 2, false>(a, st);
  // Deep layers of 24 to 32 channels per CU: 32 channels per workgroup, 8 waves up
  // to 32 tokens and 4 above (8192 x 28672 at 1/16/32/48/64 tokens
  // 37.8/40.5/49.2/61.7/70.5 us against 41.5/46.7/54.1/69.9/73.5)
  if (a.K >= 16384 && !outl && c32 <= ncu && 4 * c32 >= 3 * (int64_t)ncu) {
    if (a.T <= 32) return a.f8 ? gemv_tokens<2, 8, true>(a, st) : gemv_tokens<2, 8, false>(a, st);
    return a.f8 ? gemv_tokens<2, 4, true>(a, st) : gemv_tokens<2, 4, false>(a, st);
  }
  const bool nb2 = c32 >= ncu ? a.T > 16 : (4 * c32 >= 3 * (int64_t)ncu && a.T > 32);
  if (nb2) return a.f8 ? gemv_tokens<2, 2, true>(a, st) : gemv_tokens<2, 2, false>(a, st);
  // four waves while each CU holds a single workgroup (outlier term: two)
  if (c32 < ncu && !outl) return a.f8 ? gemv_tokens<1, 4, true>(a, st) : gemv_tokens<1, 4, false>(a, st);
  if (a.f8) return gemv_tokens<1, 2, true>(a, st);
  return gemv_tokens<1, 2, false>(a, st);
}

}  // namespace sq
