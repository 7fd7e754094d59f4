// Internal launchers of the gfx950 kernels (host side).  Arguments are already
// validated by the C ABI layer; every launcher returns hipGetLastError().
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sq {

// Largest row length the register-resident quantiser handles (256 threads x
// 8 elements x 8 chunks); longer rows take the two-pass kernel.
constexpr int64_t kQuantFastMaxK = 16384;

enum OutKind { kOutF32 = 0, kOutBF16 = 1, kOutI32 = 2 };

hipError_t launch_fill(float* p, int64_t n, float v, hipStream_t st);
hipError_t launch_fill2(float* p, float* q, int64_t n, float v, hipStream_t st);
hipError_t launch_col_absmax(const void* A, bool bf16, int64_t rows, int64_t cols, float* amax,
                             bool vec_ok, int ncu, hipStream_t st);
// Column maxima of X [T][K] and W [N][K] in one launch (running maxima into xa,
// wa); both with 16-byte aligned rows of a multiple of 16 bytes.
hipError_t launch_col_absmax_pair(const void* X, bool x_bf16, int64_t T, const void* W, bool w_bf16, int64_t N,
                                  int64_t K, float* xa, float* wa, int ncu, hipStream_t st);
// xa may alias s.
hipError_t launch_smooth_scales(const float* xa, const float* wa, int64_t K, float alpha, float* s,
                                hipStream_t st);
// s from the column maxima xa [K] (may alias s) and W [N][K], whose column
// maxima are formed inside the launch and not stored.
hipError_t launch_smooth_scales_from_w(const void* W, bool bf16, int64_t N, int64_t K, const float* xa,
                                       float alpha, float* s, bool vec_ok, hipStream_t st);
// Row quantiser modes: per-token activations (divide by s, per-row range),
// per-output-channel weights (multiply by s, per-row range; also the
// decomposition's bulk weight rows, with s a 0/1 column mask), activations against
// the range *clip (divide by s, one scale for every row); the first two with FP8
// E4M3 codes (scale = row amax / 448); and the decomposition's bulk activation
// rows (multiply by the 0/1 mask, per-row range).  Weight codes are written with
// non-temporal stores.
enum QuantMode { kQuantAct = 0, kQuantWeights = 1, kQuantActStatic = 2, kQuantActF8 = 3, kQuantWeightsF8 = 4,
                 kQuantActMasked = 5 };
hipError_t launch_quant_rows(const void* A, bool bf16, int mode, int64_t R, int64_t K,
                             const float* s, const float* clip, int8_t* Q, float* scale,
                             bool vec_ok, int ncu, hipStream_t st);
// amax[0] = max(amax[0], max over the tensor of |A_tk / s_k|)  (s may be NULL).
hipError_t launch_tensor_absmax(const void* A, bool bf16, int64_t rows, int64_t cols, const float* s,
                                float* amax, bool vec_ok, int ncu, hipStream_t st);

// Normalisation (RMSNorm, or LayerNorm when `layer`) with folded gain / bias,
// then per-token int8 of the result; mean / rstd may be NULL.
hipError_t launch_norm_quant(const void* A, bool bf16, bool layer, int64_t R, int64_t K, const float* gain,
                             const float* bias, float eps, int8_t* Q, float* scale, float* mean, float* rstd,
                             bool vec_ok, int ncu, hipStream_t st);
// Decomposition: mask[j] = 0 for the n_o columns of largest absmax (ties to the
// lower index), else 1; idx = those columns ascending.
hipError_t launch_decomp_select(const float* absmax, int64_t K, int64_t n_o, int32_t* idx, float* mask,
                                hipStream_t st);
// out[o][r] = A[r][idx[o]] (binary32)
hipError_t launch_decomp_gather(const void* A, bool bf16, int64_t rows, int64_t K, const int32_t* idx,
                                int64_t n_o, float* out, int ncu, hipStream_t st);
// out[k] = v[k] / s[k]
hipError_t launch_fold_gain(const float* v, const float* s, int64_t K, float* out, hipStream_t st);

struct GemmArgs {
  const int8_t* Xq;
  const float* xs;
  const int8_t* Wq;
  const float* ws;
  int64_t T, N, K;
  void* Y;
  int out;          // OutKind
  bool vec_store;   // Y rows allow 8/16-byte stores (N % 4 == 0, aligned base)
  // Mixed-precision decomposition (n_o > 0, float outputs only): the epilogue adds
  // sum over o (ascending, binary32) of xo[o][t] * wo[o][n]; xo is [n_o][T] and
  // wo is [n_o][N], both 16-byte aligned with T, N as leading dimensions.
  const float* xo = nullptr;
  const float* wo = nullptr;
  int64_t n_o = 0;
  // FP8 E4M3 operand bytes (binary32 accumulation; float outputs only)
  bool f8 = false;
};

// Prefill-shaped GEMM on the int8 MFMA units (K % 16 == 0, 16-byte aligned operands).
hipError_t launch_gemm_mfma(const GemmArgs& a, int ncu, hipStream_t st);
// Decode-shaped skinny GEMM (T <= 64; K % 16 == 0, 16-byte aligned operands).
hipError_t launch_gemv_mfma(const GemmArgs& a, int ncu, hipStream_t st);
// Any shape and alignment (one thread per output, scalar loads).
hipError_t launch_gemm_generic(const GemmArgs& a, hipStream_t st);

// Whether the C ABI sends a GEMM to the decode kernel rather than the tiled one.
// Up to 32 tokens always.  From 33 to 64 tokens the tiled GEMM with 64x64 tiles
// was faster on layers wider than 32 channels per CU and up to K = 11008 (10240 x
// 8192 at 48 tokens: 29.9 against 31.5 us; 28672 x 8192: 47.2 against 51.8 us);
// the decode kernel kept the lead on narrower layers, where it spreads the
// channels over all CUs (8192 x 8192: 24.1-24.7 against 29.5-30.0 us; 4096 x 4096:
// 10.6-12.1 against 15.5-15.6 us), and on deeper ones, where it splits K over two
// waves (8192 x 28672 at 33 tokens: 89.5 against 95.9 us).
inline bool use_decode_kernel(int64_t T, int64_t N, int64_t K, int ncu) {
  return T <= 32 || (T <= 64 && (K >= 12288 || (N + 31) / 32 <= ncu));
}

}  // namespace sq
