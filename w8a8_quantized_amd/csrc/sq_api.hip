// C ABI of the W8A8 layer: argument validation, kernel selection, launches.
// The semantics of each entry point are documented in include/sq.h.
#include <atomic>
#include <cmath>
#include <mutex>

#include "../../include/sq.h"
#include "kernels.h"

// Fixed scratch of the no-allocation layer call, one copy per GPU (the
// workspace of sq_w8a8_linear: int8 codes, then the per-token scales).  In host
// code `scratch` is only a handle to the symbol; its device address on each GPU
// comes from hipGetSymbolAddress and is what kernels are given.
static __device__ __align__(256) unsigned char scratch[SQ_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_ncu[kMaxDevices];   // 0 = not queried yet

// Compute units of the current device (cached; falls back to 256 if the query fails).
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int v = g_ncu[dev].load(std::memory_order_relaxed);
  if (v > 0) return v;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  g_ncu[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool in_dtype(sq_dtype t) { return t == SQ_F32 || t == SQ_BF16; }
size_t esize(sq_dtype t) { return t == SQ_BF16 ? 2 : 4; }

// Rows of `cols` elements starting at p can be read as 16-byte chunks.
bool rows_vec16(const void* p, int64_t cols, size_t es) {
  return aligned16(p) && ((uint64_t)cols * es) % 16 == 0;
}

sq_status hip_status(hipError_t e) { return e == hipSuccess ? SQ_OK : SQ_ERR_HIP; }

size_t round256(size_t v) { return (v + 255) & ~(size_t)255; }

sq_status check_gemm_args(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws,
                          int64_t T, int64_t N, int64_t K, const void* Y, sq_dtype y_t) {
  if (!Xq || !Wq || !Y) return SQ_ERR_NULL;
  if (y_t != SQ_F32 && y_t != SQ_BF16 && y_t != SQ_I32) return SQ_ERR_DTYPE;
  if (y_t != SQ_I32 && (!xs || !ws)) return SQ_ERR_NULL;
  if (T < 1 || N < 1 || K < 1 || K > SQ_MAX_K) return SQ_ERR_SHAPE;
  return SQ_OK;
}

sq_status run_gemm(const int8_t* Xq, const float* xs, const int8_t* Wq, const float* ws, int64_t T,
                   int64_t N, int64_t K, void* Y, sq_dtype y_t, hipStream_t st,
                   const float* xo = nullptr, const float* wo = nullptr, int64_t n_o = 0,
                   bool f8 = false) {
  sq::GemmArgs a;
  a.Xq = Xq; a.xs = xs; a.Wq = Wq; a.ws = ws;
  a.T = T; a.N = N; a.K = K; a.Y = Y;
  a.xo = xo; a.wo = wo; a.n_o = n_o; a.f8 = f8;
  a.out = y_t == SQ_F32 ? sq::kOutF32 : (y_t == SQ_BF16 ? sq::kOutBF16 : sq::kOutI32);
  a.vec_store = (N % 4 == 0) && aligned16(Y) && (y_t == SQ_I32 || aligned16(ws));
  const bool mfma_ok = (K % 16 == 0) && aligned16(Xq) && aligned16(Wq);
  if (!mfma_ok) return hip_status(sq::launch_gemm_generic(a, st));
  if (sq::use_decode_kernel(T, N, K, cu_count())) return hip_status(sq::launch_gemv_mfma(a, cu_count(), st));
  return hip_status(sq::launch_gemm_mfma(a, cu_count(), st));
}

sq_status run_quant_act(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* s,
                        int8_t* Xq, float* xs, hipStream_t st) {
  const bool vec = (K % 8 == 0) && rows_vec16(X, K, esize(x_t)) && aligned16(Xq);
  return hip_status(sq::launch_quant_rows(X, x_t == SQ_BF16, sq::kQuantAct, T, K, s, nullptr, Xq, xs,
                                          vec, cu_count(), st));
}

sq_status check_act_args(const void* X, sq_dtype x_t, int64_t T, int64_t K) {
  if (!X) return SQ_ERR_NULL;
  if (!in_dtype(x_t)) return SQ_ERR_DTYPE;
  if (T < 1 || K < 1) return SQ_ERR_SHAPE;
  return SQ_OK;
}

sq_status run_act_absmax(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* s,
                         float* amax, int accumulate, hipStream_t st) {
  if (!accumulate && sq::launch_fill(amax, 1, 0.0f, st) != hipSuccess) return SQ_ERR_HIP;
  const bool vec = rows_vec16(X, K, esize(x_t));
  return hip_status(sq::launch_tensor_absmax(X, x_t == SQ_BF16, T, K, s, amax, vec, cu_count(), st));
}

sq_status run_quant_static(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* s,
                           const float* clip, int8_t* Xq, float* xs, hipStream_t st) {
  const bool vec = (K % 8 == 0) && rows_vec16(X, K, esize(x_t)) && aligned16(Xq);
  return hip_status(sq::launch_quant_rows(X, x_t == SQ_BF16, sq::kQuantActStatic, T, K, s, clip, Xq,
                                          xs, vec, cu_count(), st));
}

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of the current GPU's scratch (looked up once per device), or
// nullptr if it cannot be obtained.
void* scratch_ptr() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    g_scratch[dev].store(q, std::memory_order_release);
    p = q;
  }
  return p;
}

}  // namespace

extern "C" {

const char* sq_status_string(sq_status status) {
  switch (status) {
    case SQ_OK: return "SQ_OK: success";
    case SQ_ERR_NULL: return "SQ_ERR_NULL: a required pointer is NULL";
    case SQ_ERR_SHAPE: return "SQ_ERR_SHAPE: a size is < 1 or K exceeds SQ_MAX_K";
    case SQ_ERR_ALPHA: return "SQ_ERR_ALPHA: alpha is NaN or outside [0, 1]";
    case SQ_ERR_DTYPE: return "SQ_ERR_DTYPE: dtype not accepted for this argument";
    case SQ_ERR_WORKSPACE: return "SQ_ERR_WORKSPACE: workspace missing or too small";
    case SQ_ERR_HIP: return "SQ_ERR_HIP: the HIP runtime rejected a launch";
    case SQ_ERR_ARG: return "SQ_ERR_ARG: an argument value is not accepted";
    case SQ_ERR_SCRATCH:
      return "SQ_ERR_SCRATCH: the problem needs more than the no-allocation call's fixed scratch "
             "(SQ_NOALLOC_SCRATCH_BYTES)";
  }
  return "unknown sq_status";
}

sq_status sq_col_absmax(const void* A, sq_dtype a_t, int64_t rows, int64_t cols, float* amax,
                        int accumulate, hipStream_t stream) {
  if (!A || !amax) return SQ_ERR_NULL;
  if (!in_dtype(a_t)) return SQ_ERR_DTYPE;
  if (rows < 1 || cols < 1) return SQ_ERR_SHAPE;
  if (!accumulate) {
    if (sq::launch_fill(amax, cols, 0.0f, stream) != hipSuccess) return SQ_ERR_HIP;
  }
  const bool vec = rows_vec16(A, cols, esize(a_t));
  return hip_status(sq::launch_col_absmax(A, a_t == SQ_BF16, rows, cols, amax, vec, cu_count(), stream));
}

sq_status sq_smooth_scales_from_absmax(const float* x_absmax, const float* w_absmax, int64_t K,
                                       float alpha, float* s, hipStream_t stream) {
  if (!x_absmax || !w_absmax || !s) return SQ_ERR_NULL;
  if (K < 1) return SQ_ERR_SHAPE;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ALPHA;
  return hip_status(sq::launch_smooth_scales(x_absmax, w_absmax, K, alpha, s, stream));
}

sq_status sq_smooth_scales(const void* X, sq_dtype x_t, int64_t T, const void* W, sq_dtype w_t,
                           int64_t N, int64_t K, float alpha, float* s, float* x_absmax,
                           float* w_absmax, hipStream_t stream) {
  if (!X || !W || !s) return SQ_ERR_NULL;
  if (!in_dtype(x_t) || !in_dtype(w_t)) return SQ_ERR_DTYPE;
  if (T < 1 || N < 1 || K < 1) return SQ_ERR_SHAPE;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return SQ_ERR_ALPHA;
  // X's column maxima go to x_absmax, or to s itself when they are not asked for
  float* xa = x_absmax ? x_absmax : s;
  const bool vx = rows_vec16(X, K, esize(x_t)), vw = rows_vec16(W, K, esize(w_t));
  if (w_absmax) {
    if (sq::launch_fill2(xa, w_absmax, K, 0.0f, stream) != hipSuccess) return SQ_ERR_HIP;
    if (vx && vw) {
      if (sq::launch_col_absmax_pair(X, x_t == SQ_BF16, T, W, w_t == SQ_BF16, N, K, xa, w_absmax, cu_count(),
                                     stream) != hipSuccess)
        return SQ_ERR_HIP;
    } else {
      if (sq::launch_col_absmax(X, x_t == SQ_BF16, T, K, xa, vx, cu_count(), stream) != hipSuccess ||
          sq::launch_col_absmax(W, w_t == SQ_BF16, N, K, w_absmax, vw, cu_count(), stream) != hipSuccess)
        return SQ_ERR_HIP;
    }
    return hip_status(sq::launch_smooth_scales(xa, w_absmax, K, alpha, s, stream));
  }
  // no buffer for W's maxima: each workgroup finishes the maxima of its own
  // columns over all of W and writes their factors (xa may be s: read, then written)
  if (sq::launch_fill(xa, K, 0.0f, stream) != hipSuccess ||
      sq::launch_col_absmax(X, x_t == SQ_BF16, T, K, xa, vx, cu_count(), stream) != hipSuccess)
    return SQ_ERR_HIP;
  return hip_status(sq::launch_smooth_scales_from_w(W, w_t == SQ_BF16, N, K, xa, alpha, s, vw, stream));
}

sq_status sq_quantize_weights(const void* W, sq_dtype w_t, int64_t N, int64_t K, const float* s,
                              int8_t* Wq, float* w_scale, hipStream_t stream) {
  if (!W || !Wq || !w_scale) return SQ_ERR_NULL;
  if (!in_dtype(w_t)) return SQ_ERR_DTYPE;
  if (N < 1 || K < 1) return SQ_ERR_SHAPE;
  const bool vec = (K % 8 == 0) && rows_vec16(W, K, esize(w_t)) && aligned16(Wq);
  return hip_status(sq::launch_quant_rows(W, w_t == SQ_BF16, sq::kQuantWeights, N, K, s, nullptr, Wq,
                                          w_scale, vec, cu_count(), stream));
}

sq_status sq_quant_act(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* s, int8_t* Xq,
                       float* x_scale, hipStream_t stream) {
  if (!X || !Xq || !x_scale) return SQ_ERR_NULL;
  if (!in_dtype(x_t)) return SQ_ERR_DTYPE;
  if (T < 1 || K < 1) return SQ_ERR_SHAPE;
  return run_quant_act(X, x_t, T, K, s, Xq, x_scale, stream);
}

sq_status sq_act_absmax(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* s,
                        float* amax, int accumulate, hipStream_t stream) {
  sq_status r = check_act_args(X, x_t, T, K);
  if (r != SQ_OK) return r;
  if (!amax) return SQ_ERR_NULL;
  return run_act_absmax(X, x_t, T, K, s, amax, accumulate, stream);
}

sq_status sq_quant_act_static(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* s,
                              const float* clip, int8_t* Xq, float* x_scale, hipStream_t stream) {
  sq_status r = check_act_args(X, x_t, T, K);
  if (r != SQ_OK) return r;
  if (!clip || !Xq || !x_scale) return SQ_ERR_NULL;
  return run_quant_static(X, x_t, T, K, s, clip, Xq, x_scale, stream);
}

sq_status sq_quant_act_per_tensor(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* s,
                                  float* amax, int8_t* Xq, float* x_scale, hipStream_t stream) {
  sq_status r = check_act_args(X, x_t, T, K);
  if (r != SQ_OK) return r;
  if (!amax || !Xq || !x_scale) return SQ_ERR_NULL;
  r = run_act_absmax(X, x_t, T, K, s, amax, 0, stream);
  if (r != SQ_OK) return r;
  return run_quant_static(X, x_t, T, K, s, amax, Xq, x_scale, stream);
}

sq_status sq_fold_norm_gain(const float* v, const float* s, int64_t K, float* out, hipStream_t stream) {
  if (!v || !s || !out) return SQ_ERR_NULL;
  if (K < 1) return SQ_ERR_SHAPE;
  return hip_status(sq::launch_fold_gain(v, s, K, out, stream));
}

sq_status sq_norm_quant_act(const void* X, sq_dtype x_t, int64_t T, int64_t K, sq_norm kind,
                            const float* gain, const float* bias, float eps, int8_t* Xq, float* x_scale,
                            float* mean, float* rstd, hipStream_t stream) {
  sq_status r = check_act_args(X, x_t, T, K);
  if (r != SQ_OK) return r;
  if (!gain || !Xq || !x_scale) return SQ_ERR_NULL;
  if (kind != SQ_NORM_RMS && kind != SQ_NORM_LAYER) return SQ_ERR_ARG;
  if (kind == SQ_NORM_RMS && bias) return SQ_ERR_ARG;
  if (!(eps >= 0.0f) || !std::isfinite(eps)) return SQ_ERR_ARG;
  const bool vec = (K % 8 == 0) && rows_vec16(X, K, esize(x_t)) && aligned16(Xq);
  return hip_status(sq::launch_norm_quant(X, x_t == SQ_BF16, kind == SQ_NORM_LAYER, T, K, gain, bias, eps,
                                          Xq, x_scale, mean, rstd, vec, cu_count(), stream));
}

sq_status sq_decomp_select(const float* absmax, int64_t K, int64_t n_o, int32_t* idx, float* mask,
                           hipStream_t stream) {
  if (!absmax || !mask || (n_o > 0 && !idx)) return SQ_ERR_NULL;
  if (K < 1 || n_o < 0 || n_o > K) return SQ_ERR_SHAPE;
  return hip_status(sq::launch_decomp_select(absmax, K, n_o, idx, mask, stream));
}

sq_status sq_decomp_prepare_weights(const void* W, sq_dtype w_t, int64_t N, int64_t K, const float* mask,
                                    const int32_t* idx, int64_t n_o, int8_t* Wq, float* w_scale, float* W_out,
                                    hipStream_t stream) {
  if (!W || !mask || !Wq || !w_scale || (n_o > 0 && (!idx || !W_out))) return SQ_ERR_NULL;
  if (!in_dtype(w_t)) return SQ_ERR_DTYPE;
  if (N < 1 || K < 1 || n_o < 0 || n_o > K) return SQ_ERR_SHAPE;
  const bool vec = (K % 8 == 0) && rows_vec16(W, K, esize(w_t)) && aligned16(Wq);
  if (sq::launch_quant_rows(W, w_t == SQ_BF16, sq::kQuantWeights, N, K, mask, nullptr, Wq, w_scale, vec,
                            cu_count(), stream) != hipSuccess)
    return SQ_ERR_HIP;
  return hip_status(sq::launch_decomp_gather(W, w_t == SQ_BF16, N, K, idx, n_o, W_out, cu_count(), stream));
}

sq_status sq_decomp_quant_act(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* mask,
                              const int32_t* idx, int64_t n_o, int8_t* Xq, float* x_scale, float* X_out,
                              hipStream_t stream) {
  sq_status r = check_act_args(X, x_t, T, K);
  if (r != SQ_OK) return r;
  if (!mask || !Xq || !x_scale || (n_o > 0 && (!idx || !X_out))) return SQ_ERR_NULL;
  if (n_o < 0 || n_o > K) return SQ_ERR_SHAPE;
  const bool vec = (K % 8 == 0) && rows_vec16(X, K, esize(x_t)) && aligned16(Xq);
  // per-row range and codes of X with the outlier columns multiplied by 0
  if (sq::launch_quant_rows(X, x_t == SQ_BF16, sq::kQuantActMasked, T, K, mask, nullptr, Xq, x_scale, vec,
                            cu_count(), stream) != hipSuccess)
    return SQ_ERR_HIP;
  return hip_status(sq::launch_decomp_gather(X, x_t == SQ_BF16, T, K, idx, n_o, X_out, cu_count(), stream));
}

sq_status sq_decomp_gemm(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                         const float* X_out, const float* W_out, int64_t T, int64_t N, int64_t K, int64_t n_o,
                         void* Y, sq_dtype y_t, hipStream_t stream) {
  sq_status r = check_gemm_args(Xq, x_scale, Wq, w_scale, T, N, K, Y, y_t);
  if (r != SQ_OK) return r;
  if (y_t == SQ_I32) return SQ_ERR_DTYPE;
  if (n_o < 0 || n_o > K) return SQ_ERR_SHAPE;
  if (n_o > 0 && (!X_out || !W_out)) return SQ_ERR_NULL;
  if (n_o > 0 && (!aligned16(X_out) || !aligned16(W_out))) return SQ_ERR_ARG;
  return run_gemm(Xq, x_scale, Wq, w_scale, T, N, K, Y, y_t, stream, X_out, W_out, n_o);
}

sq_status sq_quantize_weights_fp8(const void* W, sq_dtype w_t, int64_t N, int64_t K, const float* s,
                                  uint8_t* Wq, float* w_scale, hipStream_t stream) {
  if (!W || !Wq || !w_scale) return SQ_ERR_NULL;
  if (!in_dtype(w_t)) return SQ_ERR_DTYPE;
  if (N < 1 || K < 1) return SQ_ERR_SHAPE;
  const bool vec = (K % 8 == 0) && rows_vec16(W, K, esize(w_t)) && aligned16(Wq);
  return hip_status(sq::launch_quant_rows(W, w_t == SQ_BF16, sq::kQuantWeightsF8, N, K, s, nullptr,
                                          reinterpret_cast<int8_t*>(Wq), w_scale, vec, cu_count(), stream));
}

sq_status sq_quant_act_fp8(const void* X, sq_dtype x_t, int64_t T, int64_t K, const float* s, uint8_t* Xq,
                           float* x_scale, hipStream_t stream) {
  sq_status r = check_act_args(X, x_t, T, K);
  if (r != SQ_OK) return r;
  if (!Xq || !x_scale) return SQ_ERR_NULL;
  const bool vec = (K % 8 == 0) && rows_vec16(X, K, esize(x_t)) && aligned16(Xq);
  return hip_status(sq::launch_quant_rows(X, x_t == SQ_BF16, sq::kQuantActF8, T, K, s, nullptr,
                                          reinterpret_cast<int8_t*>(Xq), x_scale, vec, cu_count(), stream));
}

sq_status sq_fp8_gemm(const uint8_t* Xq, const float* x_scale, const uint8_t* Wq, const float* w_scale,
                      int64_t T, int64_t N, int64_t K, void* Y, sq_dtype y_t, hipStream_t stream) {
  const int8_t* xq = reinterpret_cast<const int8_t*>(Xq);
  const int8_t* wq = reinterpret_cast<const int8_t*>(Wq);
  sq_status r = check_gemm_args(xq, x_scale, wq, w_scale, T, N, K, Y, y_t);
  if (r != SQ_OK) return r;
  if (y_t == SQ_I32) return SQ_ERR_DTYPE;
  return run_gemm(xq, x_scale, wq, w_scale, T, N, K, Y, y_t, stream, nullptr, nullptr, 0, true);
}

sq_status sq_w8a8_gemm(const int8_t* Xq, const float* x_scale, const int8_t* Wq, const float* w_scale,
                       int64_t T, int64_t N, int64_t K, void* Y, sq_dtype y_t, hipStream_t stream) {
  sq_status r = check_gemm_args(Xq, x_scale, Wq, w_scale, T, N, K, Y, y_t);
  if (r != SQ_OK) return r;
  return run_gemm(Xq, x_scale, Wq, w_scale, T, N, K, Y, y_t, stream);
}

size_t sq_w8a8_linear_workspace_size(int64_t T, int64_t K) {
  if (T < 1 || K < 1) return 0;
  // a size that does not fit size_t is reported as SIZE_MAX, which no
  // workspace can satisfy (a wrapped product would pass the size check)
  const size_t room = (SIZE_MAX - 1024) / 2;
  if ((uint64_t)T > room / (uint64_t)K || (uint64_t)T > room / sizeof(float)) return SIZE_MAX;
  return round256((size_t)T * (size_t)K) + round256((size_t)T * sizeof(float));
}

sq_status sq_w8a8_linear(const void* X, sq_dtype x_t, const float* s, const int8_t* Wq,
                         const float* w_scale, int64_t T, int64_t N, int64_t K, void* Y, sq_dtype y_t,
                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!X || !Wq || !w_scale || !Y) return SQ_ERR_NULL;
  if (!in_dtype(x_t) || !in_dtype(y_t)) return SQ_ERR_DTYPE;
  if (T < 1 || N < 1 || K < 1 || K > SQ_MAX_K) return SQ_ERR_SHAPE;
  if (!workspace || workspace_bytes < sq_w8a8_linear_workspace_size(T, K) ||
      (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return SQ_ERR_WORKSPACE;
  int8_t* Xq = static_cast<int8_t*>(workspace);
  float* xs = reinterpret_cast<float*>(static_cast<char*>(workspace) + round256((size_t)T * (size_t)K));
  sq_status r = run_quant_act(X, x_t, T, K, s, Xq, xs, stream);
  if (r != SQ_OK) return r;
  return run_gemm(Xq, xs, Wq, w_scale, T, N, K, Y, y_t, stream);
}

sq_status sq_w8a8_linear_noalloc(const void* X, sq_dtype x_t, const float* s, const int8_t* Wq,
                                 const float* w_scale, int64_t T, int64_t N, int64_t K, void* Y, sq_dtype y_t,
                                 hipStream_t stream) {
  if (!X || !Wq || !w_scale || !Y) return SQ_ERR_NULL;
  if (!in_dtype(x_t) || !in_dtype(y_t)) return SQ_ERR_DTYPE;
  if (T < 1 || N < 1 || K < 1 || K > SQ_MAX_K) return SQ_ERR_SHAPE;
  if ((uint64_t)T > SQ_NOALLOC_SCRATCH_BYTES / (uint64_t)K ||
      sq_w8a8_linear_workspace_size(T, K) > SQ_NOALLOC_SCRATCH_BYTES)
    return SQ_ERR_SCRATCH;
  void* ws = scratch_ptr();
  if (!ws) return SQ_ERR_HIP;
  int8_t* Xq = static_cast<int8_t*>(ws);
  float* xs = reinterpret_cast<float*>(static_cast<char*>(ws) + round256((size_t)T * (size_t)K));
  sq_status r = run_quant_act(X, x_t, T, K, s, Xq, xs, stream);
  if (r != SQ_OK) return r;
  return run_gemm(Xq, xs, Wq, w_scale, T, N, K, Y, y_t, stream);
}

}  // extern "C"
