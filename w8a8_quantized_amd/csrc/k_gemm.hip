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
// consecutive output channels of one token, which the epilogue stages through
// LDS and writes as whole row segments.  Tiles of Wq and Xq are staged through an
// LDS ring of two K stages (three for the 64x128 tile), 128 bytes wide for the
// tiles with 256 rows and the 64x128 tile, 256 bytes for the 64x64 and 128x128
// tiles, one barrier per stage; the 16-byte chunk position within each LDS row is
// XOR-swizzled by the row index so that both the staging writes and the fragment
// reads (32 rows, same column) are free of bank conflicts.  Workgroups are
// remapped so that each XCD (which owns a private L2) works through a contiguous
// run of tiles, grouped 8 output-channel tiles wide, which keeps the operand
// panels it streams shared inside that L2.
//
// The same kernel serves two variants: the mixed-precision decomposition (a
// binary32 outlier-channel product added in the epilogue) and FP8 E4M3 operands
// on the FP8 matrix cores (binary32 accumulators); both are described at the
// kernel.
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "trace.h"
#include "slices.h"

namespace sq {

// Raw buffer resource over [base, base + bytes): loads whose VGPR offset is
// >= bytes return zero, which is how rows past the matrix edge become zero rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Four consecutive outputs of one row.  VEC: one 8/16-byte store (the caller
// guarantees all four exist: N % 4 == 0 and the first is in range); otherwise
// element stores of the nrem (>= 1) outputs that exist.
template <int OUT, bool VEC, typename A>
__device__ __forceinline__ void store4(void* Y, int64_t off, int nrem, const A* a, float sc_t,
                                       const float* wsv) {
  if constexpr (OUT == kOutI32) {
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
      p.x = f32x2_to_bf16x2(v[0], v[1]);
      p.y = f32x2_to_bf16x2(v[2], v[3]);
      *reinterpret_cast<uint2*>(y) = p;
      return;
    }
    for (int e = 0; e < 4 && e < nrem; ++e) y[e] = (uint16_t)f32_to_bf16(v[e]);
  }
}

// so[e] += sum over o ascending of x[o * ldx] * w[o * ldw + e], e = 0..3, one
// binary32 rounding per multiply and per add (the outlier-channel product of the
// mixed-precision decomposition).  Loads are issued OC outliers at a time, ahead
// of the dependent additions; w + o * ldw must be 16-byte aligned.
template <int OC>
__device__ __forceinline__ void outlier_sum4(const float* __restrict__ x, int64_t ldx,
                                             const float* __restrict__ w, int64_t ldw, int n_o,
                                             float* so) {
  for (int o0 = 0; o0 < n_o; o0 += OC) {
    float xv[OC];
    float4 w4[OC];
#pragma unroll
    for (int u = 0; u < OC; ++u) {
      const bool in = o0 + u < n_o;
      xv[u] = in ? x[(int64_t)(o0 + u) * ldx] : 0.0f;
      w4[u] = in ? *reinterpret_cast<const float4*>(w + (int64_t)(o0 + u) * ldw) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int u = 0; u < OC; ++u) {
      if (o0 + u < n_o) {
        so[0] = so[0] + xv[u] * w4[u].x;
        so[1] = so[1] + xv[u] * w4[u].y;
        so[2] = so[2] + xv[u] * w4[u].z;
        so[3] = so[3] + xv[u] * w4[u].w;
      }
    }
  }
}

// Element stores of the nrem (>= 1) outputs that exist, each the dequantised
// value plus its outlier-channel product (float outputs only).
template <int OUT, typename A>
__device__ __forceinline__ void store4o(void* Y, int64_t off, int nrem, const A* a, float sc_t,
                                        const float* wsv, const float* so) {
  for (int e = 0; e < 4 && e < nrem; ++e) {
    const float v = (float)a[e] * (sc_t * wsv[e]) + so[e];
    if (OUT == kOutF32) static_cast<float*>(Y)[off + e] = v;
    else static_cast<uint16_t*>(Y)[off + e] = (uint16_t)f32_to_bf16(v);
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

// s_waitcnt immediate for "vmcnt <= n" (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14; expcnt 6:4 left at 7; lgkmcnt 11:8 at 15, or at 0 with kLgkm0).
constexpr int vmcnt_enc(int n) { return 0x0F70 | (n & 15) | (((n >> 4) & 3) << 14); }
[[maybe_unused]] constexpr int kLgkm0 = ~0x0F00;

// Requires K % 16 == 0, (N + BN) * K < 2^31 and (T + BT) * K < 2^31 (the host
// splits larger problems), 16-byte aligned Xq and Wq.
//
// Main loop.  A STAGES-deep ring of LDS stages, each holding BN rows of Wq and
// BT rows of Xq, BK bytes wide.  Stages are filled by direct-to-LDS buffer loads
// (one 1 KB wave instruction per 64/CPR rows: lane l deposits 16 bytes at
// slot l of the instruction's 1 KB block, so each lane fetches the logical
// chunk that belongs at its slot under the XOR swizzle).  Fragments of step q+1
// are read from LDS while the MFMAs of step q run; the per-stage barrier sits
// after all (16-wave tile) or half (the others) of the last step's MFMAs.  The
// barrier is a bare s_barrier
// preceded by this wave's own "vmcnt <= loads of later stages" wait: a fenced
// barrier would also wait for the later stages still in flight.
//
// Epilogue (VEC).  Each wave stages 32 token rows x WTN outputs at a time in
// LDS (rows padded by 16 bytes) and writes them back as row-contiguous 16-byte
// stores, so every store instruction covers whole 256/512-byte row segments.
//
// PERSIST (int8 or FP8, no outlier term, staged epilogue): the grid is one workgroup
// per CU and each walks tiles blockIdx.x, + gridDim.x, ... in the same tile
// order.  The staging rows sit past ring stage 0, and once a tile's main loop
// is done the next tile's first stage is issued into stage 0, so its load
// overlaps the epilogue; a barrier after the epilogue frees the staging rows
// for the next tile's later stages.  The stage waits count this wave's vector
// memory operations in issue order, the epilogue's stores included.
//
// OUTL (mixed-precision decomposition, mercemay.com "Activation Outlier Channels
// and Mixed-Precision Decomposition", section "Decomposition"): the float
// epilogue value gets the binary32 product of the outlier channels added,
//   y = fl32(fl32(acc) * fl32(xs * ws)) + (sum over o ascending of xo[o][t] * wo[o][n]).
// When they fit in the freed operand ring, the tile's outlier operands are first
// copied into LDS, and each lane forms the sums of a 32-channel block's four
// channel quadruples in one pass over the outliers; otherwise it reads xo / wo
// from global memory per quadruple.
//
// F8 (FP8 E4M3 operands, inferenceinterviews.com formats paragraph): the same
// byte tiles feed v_mfma_f32_32x32x64_f8f6f4 with binary32 accumulators (the
// compiler selects the unscaled instruction for the scaled builtin with zero
// scale operands; on the GPU it gives the bits of the scaled form with E8M0 unit
// scales, 127, on 4M random outputs, and issues without the scale operands).  One MFMA takes, per lane, the two 16-byte chunks that
// two consecutive int8 k-steps would take, for A and B alike, so every product
// pairs the same k.  FP8 runs 8 waves of 64x128 per 256x256 tile (the operands
// are twice as wide per lane, and the 16-wave layout would spill); the A
// fragments alternate between two register slots and each B fragment is re-read
// for the next step once its last MFMA of the step has issued, so the reads
// overlap the MFMAs within the 256 registers of two waves per SIMD (measured 4%
// faster on 8192^3 than reading each step's operands before its MFMAs).
template <int BN, int BT, int BK, int WN, int WT, int STAGES, int OUT, bool VEC, bool OUTL, bool F8,
          bool PERSIST = false>
__global__ __launch_bounds__(WN* WT * 64) void gemm_i8_mfma_kernel(
    const int8_t* __restrict__ Xq, const float* __restrict__ xs, const int8_t* __restrict__ Wq,
    const float* __restrict__ ws, int T, int N, int K, void* __restrict__ Y, int64_t ldy,
    int tiles_n, int tiles_t, const float* __restrict__ xo, int64_t ldxo,
    const float* __restrict__ wo, int64_t ldwo, int n_o) {
  // The body exists only in the device pass (the host pass needs just the
  // launch stub, and its front end cannot take the device scheduling builtins).
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NW = WN * WT;
  constexpr int CPR = BK / 16;                 // 16-byte chunks per LDS row
  constexpr int RPB = 16 / CPR;                // rows sharing one 256-byte bank line
  constexpr int ROWS_PER_INSN = 64 / CPR;      // rows one wave-wide DMA load covers
  constexpr int WTN = BN / WN, WTT = BT / WT;  // wave tile
  constexpr int RN = WTN / 32, RT = WTT / 32;  // 32x32 MFMA blocks per wave
  constexpr int KK = BK / 32;                  // MFMA k-steps per stage
  constexpr int A_INSN = BN / ROWS_PER_INSN / NW, B_INSN = BT / ROWS_PER_INSN / NW;
  constexpr int STAGE_BYTES = (BN + BT) * BK;
  constexpr int PER = A_INSN + B_INSN;         // DMA loads per stage per wave
  static_assert(A_INSN * ROWS_PER_INSN * NW == BN && B_INSN * ROWS_PER_INSN * NW == BT, "tile/waves");
  static_assert(KK % 2 == 0 && STAGES >= 2, "pipeline shape");
  static_assert(!PERSIST || (VEC && !OUTL), "persistent form: no outlier term, LDS-staged epilogue");
  // LDS-staged epilogue: each wave stages 32 token rows of EW outputs; all RN
  // column blocks of the wave tile at once when that fits in the operand ring,
  // else one 32-column block at a time.  The persistent form keeps the staging
  // rows clear of ring stage 0, which receives the next tile's first stage
  // while the epilogue runs.
  constexpr int OB = (OUT == kOutBF16) ? 2 : 4;
  constexpr int EI = (NW * 32 * (WTN * OB + 16) <= STAGES * STAGE_BYTES) ? RN : 1;
  constexpr int EW = EI * 32;                // outputs per staged row
  constexpr int ROWB = EW * OB + 16;         // padded staging row
  constexpr int EOFF = PERSIST ? STAGE_BYTES : 0;
  constexpr int LDS_BYTES =
      EOFF + NW * 32 * ROWB > STAGES * STAGE_BYTES ? EOFF + NW * 32 * ROWB : STAGES * STAGE_BYTES;
  __shared__ __attribute__((aligned(1024))) int8_t lds[LDS_BYTES];

  // Persistent form: this workgroup takes tiles blockIdx.x, + gridDim.x, ...
  const int total_tiles = tiles_n * tiles_t;
  int tile = blockIdx.x;
  bool stage0_issued = false;   // the tile's first stage went out during the previous epilogue
  for (;;) {
  int tn, tt;
  tile_coords(tile, PERSIST ? total_tiles : (int)gridDim.x, tiles_n, tiles_t, tn, tt);
  const int n0 = tn * BN, t0 = tt * BT;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wn = wave % WN, wt = wave / WN;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(Wq, N * K);
  const __amdgpu_buffer_rsrc_t rsB = make_rsrc(Xq, T * K);

  // DMA source offsets: LDS row r of an instruction block, physical chunk pc,
  // holds logical chunk pc ^ swz(r).
  const int lrow = lane / CPR, pc = lane % CPR;
  int a_off[A_INSN], b_off[B_INSN], a_ch[A_INSN], b_ch[B_INSN];
  auto set_offsets = [&](int n0_, int t0_) {
#pragma unroll
    for (int p = 0; p < A_INSN; ++p) {
      const int row = (wave * A_INSN + p) * ROWS_PER_INSN + lrow;
      a_ch[p] = (pc ^ ((row / RPB) % CPR)) * 16;
      a_off[p] = (n0_ + row) * K + a_ch[p];
    }
#pragma unroll
    for (int p = 0; p < B_INSN; ++p) {
      const int row = (wave * B_INSN + p) * ROWS_PER_INSN + lrow;
      b_ch[p] = (pc ^ ((row / RPB) % CPR)) * 16;
      b_off[p] = (t0_ + row) * K + b_ch[p];
    }
  };
  set_offsets(n0, t0);
  // The whole byte offset goes in the VGPR operand: the buffer range check
  // covers that operand (not the scalar one), so rows past the edge and masked
  // K-tail chunks (sent to kOob) arrive as zeros and never leave the allocation.
  constexpr int kOob = 0x7FFFFFF0;
  auto issue = [&](int buf, int k0) {
    int8_t* L = lds + buf * STAGE_BYTES;
    const int kv = K - k0;
#pragma unroll
    for (int p = 0; p < A_INSN; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsA, (__attribute__((address_space(3))) void*)(L + (wave * A_INSN + p) * 1024), 16,
          a_ch[p] < kv ? a_off[p] + k0 : kOob, 0, 0, 0);
#pragma unroll
    for (int p = 0; p < B_INSN; ++p)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsB, (__attribute__((address_space(3))) void*)(L + BN * BK + (wave * B_INSN + p) * 1024), 16,
          b_ch[p] < kv ? b_off[p] + k0 : kOob, 0, 0, 0);
  };

  // Fragment reads: rows wn*WTN + i*32 + fr (A) and wt*WTT + j*32 + fr (B).  The
  // block offsets are multiples of 16 rows, so the swizzle depends on fr only.
  const int fr = lane & 31, fc = lane >> 5;
  const int sw = (fr / RPB) % CPR;
  const int a_base = (wn * WTN + fr) * BK;
  const int b_base = BN * BK + (wt * WTT + fr) * BK;
  int cofs[KK];
#pragma unroll
  for (int kk = 0; kk < KK; ++kk) cofs[kk] = ((kk * 2 + fc) ^ sw) * 16;

  using AccT = std::conditional_t<F8, v16f, v16i>;
  using AccE = std::conditional_t<F8, float, int>;
  static_assert(!F8 || OUT != kOutI32, "FP8 accumulators are binary32");
  AccT acc[RN][RT];
#pragma unroll
  for (int i = 0; i < RN; ++i)
#pragma unroll
    for (int j = 0; j < RT; ++j) acc[i][j] = AccT{};

  v4i fa[2][RN], fb[2][RT];
  auto read_frags = [&](int slot, const int8_t* L, int kk) {
#pragma unroll
    for (int i = 0; i < RN; ++i) fa[slot][i] = *reinterpret_cast<const v4i*>(L + a_base + cofs[kk] + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < RT; ++j) fb[slot][j] = *reinterpret_cast<const v4i*>(L + b_base + cofs[kk] + j * 32 * BK);
  };
  auto mfmas = [&](int slot, int first, int count) {
    if constexpr (!F8) {
#pragma unroll
      for (int q = 0; q < RN * RT; ++q) {
        if (q < first || q >= first + count) continue;
        const int i = q / RT, j = q % RT;
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[slot][i], fb[slot][j], acc[i][j], 0, 0, 0);
      }
    }
  };
  // FP8: the operands of one 64-deep step are the chunks of int8 k-steps 2q and
  // 2q + 1, read straight into 8-register operands.  The A fragments have two
  // slots; each B fragment is re-read for the next step as soon as the last MFMA
  // of this step that uses it has issued.
  v8i ga[F8 ? 2 : 1][F8 ? RN : 1], gb[F8 ? RT : 1];
  auto frag8 = [&](const int8_t* L, int base, int q) {
    return __builtin_shufflevector(*reinterpret_cast<const v4i*>(L + base + cofs[2 * q]),
                                   *reinterpret_cast<const v4i*>(L + base + cofs[2 * q + 1]), 0, 1, 2, 3, 4, 5,
                                   6, 7);
  };
  auto readA8 = [&](int slot, const int8_t* L, int q) {
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < RN; ++i) ga[slot][i] = frag8(L, a_base + i * 32 * BK, q);
    }
  };
  auto readB8 = [&](int j, const int8_t* L, int q) {
    if constexpr (F8) gb[j] = frag8(L, b_base + j * 32 * BK, q);
  };
  // the MFMAs of one B fragment (column block j of the wave tile)
  auto col8 = [&](int slot, int j) {
    if constexpr (F8) {
#pragma unroll
      for (int i = 0; i < RN; ++i)
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga[slot][i], gb[j], acc[i][j], 0, 0, 0, 0, 0, 0);
    }
  };
  // wait until at most `later` stages of this wave's DMA loads are in flight
  // (and, for wait_vm_lds, its LDS reads are complete)
  // (the counter limit is 63 loads; deeper rings wait conservatively)
  auto wait_vm = [&](int later) {
    static_assert(PER <= 63, "loads per stage");
    if (later >= 7 && 7 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(7 * PER <= 63 ? 7 * PER : 0));
    else if (later >= 6 && 6 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(6 * PER <= 63 ? 6 * PER : 0));
    else if (later >= 5 && 5 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(5 * PER <= 63 ? 5 * PER : 0));
    else if (later >= 4 && 4 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(4 * PER <= 63 ? 4 * PER : 0));
    else if (later >= 3 && 3 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(3 * PER <= 63 ? 3 * PER : 0));
    else if (later >= 2 && 2 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * PER <= 63 ? 2 * PER : 0));
    else if (later >= 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(PER));
    else __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
  };
  auto wait_vm_lds = [&](int later) {
    if (later >= 7 && 7 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(7 * PER <= 63 ? 7 * PER : 0) & kLgkm0);
    else if (later >= 6 && 6 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(6 * PER <= 63 ? 6 * PER : 0) & kLgkm0);
    else if (later >= 5 && 5 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(5 * PER <= 63 ? 5 * PER : 0) & kLgkm0);
    else if (later >= 4 && 4 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(4 * PER <= 63 ? 4 * PER : 0) & kLgkm0);
    else if (later >= 3 && 3 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(3 * PER <= 63 ? 3 * PER : 0) & kLgkm0);
    else if (later >= 2 && 2 * PER <= 63) __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * PER <= 63 ? 2 * PER : 0) & kLgkm0);
    else if (later >= 1) __builtin_amdgcn_s_waitcnt(vmcnt_enc(PER) & kLgkm0);
    else __builtin_amdgcn_s_waitcnt(vmcnt_enc(0) & kLgkm0);
  };
  auto bar = [&] {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };

  const int nst = (K + BK - 1) / BK;
#pragma unroll
  for (int s = 0; s < STAGES; ++s)
    if (s < nst && !(s == 0 && stage0_issued)) issue(s, s * BK);
  wait_vm(nst - 1 < STAGES - 1 ? nst - 1 : STAGES - 1);
  bar();

  if constexpr (F8) {
    // As in the int8 schedule below, the last step of a stage runs half of its
    // MFMAs, meets the other waves at the stage barrier, reads the next stage's
    // first operands, then runs the other half.  The stage body has no branches
    // (the last stages are separate copies): the MFMAs have no side effects, and
    // across a branch the compiler would move them away from their reads.
    constexpr int Q = KK / 2;
    constexpr int H = RT / 2;   // B fragments whose MFMAs precede the stage barrier
    static_assert(Q % 2 == 0, "A slots alternate within a stage");
    auto stage8 = [&](int s, auto more_c, auto issue_c) {
      constexpr bool MORE = decltype(more_c)::value;   // a next stage follows
      constexpr bool ISSUE = decltype(issue_c)::value; // stage s + STAGES exists
      const int8_t* L = lds + (s % STAGES) * STAGE_BYTES;
      const int8_t* Ln = lds + ((s + 1) % STAGES) * STAGE_BYTES;
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int cur = q & 1, nxt = cur ^ 1;
        if (q + 1 < Q) {
#pragma unroll
          for (int j = 0; j < RT; ++j) {
            col8(cur, j);
            __builtin_amdgcn_sched_barrier(0);
            if (j == 0) readA8(nxt, L, q + 1);
            readB8(j, L, q + 1);
            __builtin_amdgcn_sched_barrier(0);
          }
        } else {
#pragma unroll
          for (int j = 0; j < H; ++j) col8(cur, j);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (MORE) {
            wait_vm_lds(ISSUE ? STAGES - 2 : nst - 2 - s);
            bar();
            if constexpr (ISSUE) issue(s % STAGES, (s + STAGES) * BK);
            readA8(nxt, Ln, 0);
#pragma unroll
            for (int j = 0; j < H; ++j) readB8(j, Ln, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int j = H; j < RT; ++j) {
            col8(cur, j);
            __builtin_amdgcn_sched_barrier(0);
            if constexpr (MORE) readB8(j, Ln, 0);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
    };
    readA8(0, lds, 0);
#pragma unroll
    for (int j = 0; j < RT; ++j) readB8(j, lds, 0);
    int s = 0;
    for (; s + STAGES < nst; ++s) stage8(s, std::true_type{}, std::true_type{});
    for (; s + 1 < nst; ++s) stage8(s, std::true_type{}, std::false_type{});
    stage8(s, std::false_type{}, std::false_type{});
    // keep the last stage's MFMAs here: sunk into the epilogue, next to its
    // cached channel scales, they made the compiler spill
#pragma unroll
    for (int i = 0; i < RN; ++i)
#pragma unroll
      for (int j = 0; j < RT; ++j) asm volatile("" : "+v"(acc[i][j]));
  } else {
    // Per stage: KK k-steps; each step's MFMAs run while the next step's
    // fragments are read.  The last step runs PRE of its MFMAs, meets the other
    // waves at the stage barrier (stage s + 1 must have landed, later ones may
    // stay in flight; this wave's fragment reads of stage s must be complete),
    // issues stage s + STAGES into the freed slot and reads stage s + 1's first
    // fragments, then runs the rest.  With one or two waves per SIMD (the 128x128
    // and 64x64 tiles) half of the MFMAs after the barrier cover those reads
    // (512x4096x4096 2-4% faster); with four (16 waves of 256x256) the other
    // waves cover them, and all before the barrier measured ~1% faster on 8192^3.
    // As for FP8, the stage body has no branches, so the compiler keeps the
    // MFMAs where they are written.
    constexpr int PRE = NW >= 16 ? RN * RT : RN * RT / 2;
    auto stage = [&](int s, auto more_c, auto issue_c) {
      constexpr bool MORE = decltype(more_c)::value;   // a next stage follows
      constexpr bool ISSUE = decltype(issue_c)::value; // stage s + STAGES exists
      const int8_t* L = lds + (s % STAGES) * STAGE_BYTES;
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        const int cur = kk & 1, nxt = cur ^ 1;
        if (kk + 1 < KK) {
          read_frags(nxt, L, kk + 1);
          mfmas(cur, 0, RN * RT);
          // interleave the next step's fragment reads with this step's MFMAs
#pragma unroll
          for (int q = 0; q < RN + RT; ++q) {
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one LDS read
            __builtin_amdgcn_sched_group_barrier(0x008, (RN * RT) / (RN + RT), 0);   // MFMAs
          }
          __builtin_amdgcn_sched_barrier(0);
        } else {
          mfmas(cur, 0, PRE);
          __builtin_amdgcn_sched_barrier(0);
          if constexpr (MORE) {
            wait_vm_lds(ISSUE ? STAGES - 2 : nst - 2 - s);
            bar();
            if constexpr (ISSUE) issue(s % STAGES, (s + STAGES) * BK);
            read_frags(nxt, lds + ((s + 1) % STAGES) * STAGE_BYTES, 0);
          }
          __builtin_amdgcn_sched_barrier(0);
          mfmas(cur, PRE, RN * RT - PRE);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    };
    read_frags(0, lds, 0);
    int s = 0;
    for (; s + STAGES < nst; ++s) stage(s, std::true_type{}, std::true_type{});
    for (; s + 1 < nst; ++s) stage(s, std::true_type{}, std::false_type{});
    stage(s, std::false_type{}, std::false_type{});
  }

  int next_tile = total_tiles;
  if (VEC) {
    // ---- epilogue through LDS (requires N % (16 / output bytes) == 0, 16-byte aligned Y, ws)
    __syncthreads();   // every wave is done with the operand ring
    if constexpr (PERSIST) {
      // the next tile's first stage streams into ring stage 0 during the epilogue
      next_tile = tile + (int)gridDim.x;
      if (next_tile < total_tiles) {
        int ntn, ntt;
        tile_coords(next_tile, total_tiles, tiles_n, tiles_t, ntn, ntt);
        set_offsets(ntn * BN, ntt * BT);
        issue(0, 0);
      }
    }
    constexpr int CPRO = EW * OB / 16;         // 16-byte chunks per output row
    constexpr int RPI = 64 / CPRO;             // output rows per wave instruction
    static_assert(EOFF + NW * 32 * ROWB <= LDS_BYTES, "epilogue staging does not fit");
    int8_t* E = lds + EOFF + wave * (32 * ROWB);
    // Outlier operands of this tile (decomposition): the token values
    // xo[o][t0 .. t0 + BT) and channel values wo[o][n0 .. n0 + BN) are copied
    // into the LDS past the staging rows when they fit (zero past T or N), so
    // the epilogue reads them from LDS; else it reads them from xo / wo.
    constexpr int OFREE = LDS_BYTES - EOFF - NW * 32 * ROWB;
    float* oxl = reinterpret_cast<float*>(lds + EOFF + NW * 32 * ROWB);   // [n_o][BT]
    float* owl = oxl + (OUTL ? n_o : 0) * BT;                       // [n_o][BN]
    const bool ostage = OUTL && n_o > 0 && n_o * (BT + BN) * 4 <= OFREE;
    if (ostage) {
      const int nx = n_o * BT, ntot = nx + n_o * BN;
      for (int q0 = threadIdx.x; q0 < ntot; q0 += 4 * NW * 64) {
        float v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int q = q0 + u * NW * 64;
          v[u] = 0.0f;
          if (q < nx) {
            const int o = q / BT, tt = q - o * BT;
            if (t0 + tt < T) v[u] = xo[(int64_t)o * ldxo + t0 + tt];
          } else if (q < ntot) {
            const int o = (q - nx) / BN, nn = q - nx - o * BN;
            if (n0 + nn < N) v[u] = wo[(int64_t)o * ldwo + n0 + nn];
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (q0 + u * NW * 64 < ntot) oxl[q0 + u * NW * 64] = v[u];
      }
      __syncthreads();
    }
    // channel scales held across the token blocks (re-read per block instead
    // when the outlier term needs the registers)
    float wsq[RN][4][4];
    if (OUT != kOutI32 && !OUTL) {
#pragma unroll
      for (int i = 0; i < RN; ++i)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WTN + i * 32 + 8 * g + 4 * fc;
          const float4 w4 = (n < N) ? *reinterpret_cast<const float4*>(ws + n) : make_float4(0.f, 0.f, 0.f, 0.f);
          wsq[i][g][0] = w4.x; wsq[i][g][1] = w4.y; wsq[i][g][2] = w4.z; wsq[i][g][3] = w4.w;
        }
    }
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const int t_l = t0 + wt * WTT + j * 32 + fr;
      const float sc = (OUT != kOutI32 && t_l < T) ? xs[t_l] : 0.0f;
#pragma unroll
      for (int ib = 0; ib < RN; ib += EI) {
        // LDS accesses of one wave complete in order, so this round's writes
        // follow the previous round's reads of the same staging rows.
#pragma unroll
        for (int i = ib; i < ib + EI; ++i) {
          // staged outlier sums of this lane's four channel quadruples of block
          // i for token t_l: one pass over the outliers in ascending order, one
          // binary32 rounding per multiply and per add
          float so4[4][4];
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) so4[g][e] = 0.0f;
          if (OUTL && ostage) {
            const int tt = t_l - t0, nn = wn * WTN + i * 32 + 4 * fc;
            for (int o = 0; o < n_o; ++o) {
              const float x = oxl[o * BT + tt];
              float4 w4[4];
#pragma unroll
              for (int g = 0; g < 4; ++g) w4[g] = *reinterpret_cast<const float4*>(owl + o * BN + nn + 8 * g);
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                so4[g][0] = so4[g][0] + x * w4[g].x;
                so4[g][1] = so4[g][1] + x * w4[g].y;
                so4[g][2] = so4[g][2] + x * w4[g].z;
                so4[g][3] = so4[g][3] + x * w4[g].w;
              }
            }
          }
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            int8_t* dst = E + fr * ROWB + ((i - ib) * 32 + 8 * g + 4 * fc) * OB;
            if constexpr (OUT == kOutI32) {
              *reinterpret_cast<v4i*>(dst) =
                  v4i{acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
            } else {
              float v[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if (OUTL) {
                  const int nw = n0 + wn * WTN + i * 32 + 8 * g + 4 * fc;
                  wsq[i][g][e] = nw < N ? ws[nw + e] : 0.0f;
                }
                v[e] = (float)acc[i][j][4 * g + e] * (sc * wsq[i][g][e]);
              }
              if (OUTL) {
                const int n = n0 + wn * WTN + i * 32 + 8 * g + 4 * fc;
                float so[4] = {so4[g][0], so4[g][1], so4[g][2], so4[g][3]};
                // unstaged: chunks of 4 keep the 16-wave tile within its 128 registers
                if (!ostage && t_l < T && n < N) outlier_sum4<(NW > 8 ? 4 : 8)>(xo + t_l, ldxo, wo + n, ldwo, n_o, so);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] = v[e] + so[e];
              }
              if (OUT == kOutF32) {
                *reinterpret_cast<float4*>(dst) = make_float4(v[0], v[1], v[2], v[3]);
              } else {
                uint2 p;
                p.x = f32x2_to_bf16x2(v[0], v[1]);
                p.y = f32x2_to_bf16x2(v[2], v[3]);
                *reinterpret_cast<uint2*>(dst) = p;
              }
            }
          }
        }
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
          const int row = it * RPI + lane / CPRO, ch = lane % CPRO;
          const v4i val = *reinterpret_cast<const v4i*>(E + row * ROWB + ch * 16);
          const int t = t0 + wt * WTT + j * 32 + row;
          const int n = n0 + wn * WTN + ib * 32 + ch * (16 / OB);
          if (t < T && n < N) *reinterpret_cast<v4i*>(static_cast<int8_t*>(Y) + ((int64_t)t * ldy + n) * OB) = val;
        }
      }
    }
  } else {
    // ---- direct epilogue, element stores (any N, any alignment)
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const int t = t0 + wt * WTT + j * 32 + fr;
      if (t >= T) continue;
      const float sc = (OUT == kOutI32) ? 0.0f : xs[t];
#pragma unroll
      for (int i = 0; i < RN; ++i) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * WTN + i * 32 + 8 * g + 4 * fc;
          if (n >= N) continue;
          const AccE a4[4] = {acc[i][j][4 * g], acc[i][j][4 * g + 1], acc[i][j][4 * g + 2], acc[i][j][4 * g + 3]};
          float wsv[4] = {0.f, 0.f, 0.f, 0.f};
          if (OUT != kOutI32)
            for (int e = 0; e < 4; ++e) wsv[e] = (n + e < N) ? ws[n + e] : 0.0f;
          if (OUTL) {
            float so[4] = {0.f, 0.f, 0.f, 0.f};
            for (int o = 0; o < n_o; ++o) {
              const float xv = xo[(int64_t)o * ldxo + t];
              for (int e = 0; e < 4; ++e)
                if (n + e < N) so[e] = so[e] + xv * wo[(int64_t)o * ldwo + n + e];
            }
            store4o<OUT>(Y, (int64_t)t * ldy + n, N - n, a4, sc, wsv, so);
          } else {
            store4<OUT, false>(Y, (int64_t)t * ldy + n, N - n, a4, sc, wsv);
          }
        }
      }
    }
  }
  if constexpr (!PERSIST) {
    break;
  } else {
    if (next_tile >= total_tiles) break;
    // every wave is done with its staging rows, which ring stages >= 1 reuse
    __syncthreads();
    tile = next_tile;
    stage0_issued = true;
  }
  }   // tile loop
#endif
}

template <int BN, int BT, int BK, int WN, int WT, int ST, bool VEC, bool F8, bool PERSIST = false>
static void launch_out(int out, bool outl, dim3 grid, dim3 block, hipStream_t st, const int8_t* Xq,
                       const float* xs, const int8_t* Wq, const float* ws, int T, int N, int K, void* Y,
                       int64_t ldy, int tiles_n, int tiles_t, const float* xo, int64_t ldxo, const float* wo,
                       int64_t ldwo, int n_o) {
  SQ_TRACE("gemm_i8_mfma tile %dx%d (channels x tokens) k-stage %d B, waves %dx%d, %d stages, out %s%s%s%s, "
           "T %d N %d K %d, %dx%d tiles, grid %u x %u threads",
           BN, BT, BK, WN, WT, ST, out == kOutF32 ? "f32" : out == kOutBF16 ? "bf16" : "i32",
           outl ? ", outlier term" : "", F8 ? ", fp8" : "", PERSIST ? ", persistent" : "", T, N, K, tiles_n,
           tiles_t, grid.x, block.x);
#define SQ_GEMM_LAUNCH(O, L, F)                                                                                  \
  hipLaunchKernelGGL((gemm_i8_mfma_kernel<BN, BT, BK, WN, WT, ST, O, VEC, L, F, PERSIST>), grid, block, 0, st, Xq, \
                     xs, Wq, ws, T, N, K, Y, ldy, tiles_n, tiles_t, xo, ldxo, wo, ldwo, n_o)
  if constexpr (PERSIST && F8) {
    (void)outl;
    if (out == kOutF32) SQ_GEMM_LAUNCH(kOutF32, false, true);
    else SQ_GEMM_LAUNCH(kOutBF16, false, true);
    return;
  } else if constexpr (PERSIST) {   // no outlier term
    (void)outl;
    if (out == kOutF32) SQ_GEMM_LAUNCH(kOutF32, false, false);
    else if (out == kOutBF16) SQ_GEMM_LAUNCH(kOutBF16, false, false);
    else SQ_GEMM_LAUNCH(kOutI32, false, false);
    return;
  } else if constexpr (F8) {   // FP8 operands: float outputs, no outlier term
    if (out == kOutF32) SQ_GEMM_LAUNCH(kOutF32, false, true);
    else SQ_GEMM_LAUNCH(kOutBF16, false, true);
    return;
  } else {
  switch (out) {
    case kOutF32:
      if (outl) SQ_GEMM_LAUNCH(kOutF32, true, false); else SQ_GEMM_LAUNCH(kOutF32, false, false);
      break;
    case kOutBF16:
      if (outl) SQ_GEMM_LAUNCH(kOutBF16, true, false); else SQ_GEMM_LAUNCH(kOutBF16, false, false);
      break;
    default:
      SQ_GEMM_LAUNCH(kOutI32, false, false);
      break;
  }
  }
#undef SQ_GEMM_LAUNCH
}

template <int BN, int BT, int BK, int WN, int WT, int ST, bool F8 = false, bool PERSIST = false>
static hipError_t gemm_cfg(const GemmArgs& a, hipStream_t st, int ncu = 0) {
  // Split so that every operand slice handed to one launch spans < 2^31 bytes
  // (32-bit buffer offsets), counting one tile of overhang past the edge.
  const int64_t n_chunk = rows_per_slice(a.K, BN);
  const int64_t t_chunk = rows_per_slice(a.K, BT);
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
      const bool outl = a.n_o > 0 && a.out != kOutI32 && !a.f8;
      const float* xo = outl ? a.xo + tb : nullptr;
      const float* wo = outl ? a.wo + nb : nullptr;
      void* Y = static_cast<char*>(a.Y) + (tb * a.N + nb) * osz;
      // a column slice of Y keeps 16-byte alignment only if nb is a multiple of 4
      // the LDS-staged epilogue writes 16-byte row chunks: N must be a multiple of
      // 16 / (output bytes) and the column slice must keep 16-byte alignment
      const int per16 = a.out == kOutBF16 ? 8 : 4;
      const bool vs = a.vec_store && a.N % per16 == 0 && nb % per16 == 0;
      const int K = (int)a.K;
      // persistent form (one workgroup per CU walking its tiles): no outlier
      // term, LDS-staged epilogue only
      bool done = false;
      if constexpr (PERSIST) {
        if (vs && !outl && ncu > 0 && tiles_n * tiles_t > ncu) {
          launch_out<BN, BT, BK, WN, WT, ST, true, F8, true>(a.out, false, dim3(ncu), block, st, Xq, xs, Wq, ws, T, N,
                                                            K, Y, a.N, tiles_n, tiles_t, nullptr, a.T, nullptr, a.N, 0);
          done = true;
        }
      }
      if (done) {
      } else if (vs) {
        launch_out<BN, BT, BK, WN, WT, ST, true, F8>(a.out, outl, grid, block, st, Xq, xs, Wq, ws, T, N, K, Y, a.N,
                                                   tiles_n, tiles_t, xo, a.T, wo, a.N, (int)a.n_o);
      } else {
        launch_out<BN, BT, BK, WN, WT, ST, false, F8>(a.out, outl, grid, block, st, Xq, xs, Wq, ws, T, N, K, Y, a.N,
                                                    tiles_n, tiles_t, xo, a.T, wo, a.N, (int)a.n_o);
      }
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}

hipError_t launch_gemm_mfma(const GemmArgs& a, int ncu, hipStream_t st) {
  // Up to 64 tokens (the shapes the decode kernel does not take): one 64-token
  // tile reads every weight tile once, so 64x64 tiles, whatever the layer's width.
  if (a.T <= 64) {
    if (a.f8) return gemm_cfg<64, 64, 256, 2, 2, 2, true>(a, st);
    return gemm_cfg<64, 64, 256, 2, 2, 2>(a, st);
  }
  if (a.f8) {
    // 8 waves of 64 x 128: the FP8 step's 8-register operands and their
    // second slot need ~240 registers per wave, more than the 16-wave tile allows.
    // More tiles than CUs: the persistent form, as for int8 (1.2% faster on
    // 8192^3 and 2048x16384x4096).
    const int64_t big8 = ((a.N + 255) / 256) * ((a.T + 255) / 256);
    if (big8 >= ncu) return gemm_cfg<256, 256, 128, 4, 2, 2, true, true>(a, st, ncu);
    // smaller problems: the int8 choice of tiles
    if (4 * big8 >= 3 * ncu) return gemm_cfg<256, 256, 128, 4, 2, 2, true>(a, st);
    if (a.T <= 128 && (a.N + 127) / 128 >= (3 * ncu) / 4) return gemm_cfg<128, 128, 256, 2, 2, 2, true>(a, st);
    if (a.T <= 128 && (a.N + 63) / 64 >= (3 * ncu) / 4) return gemm_cfg<64, 128, 128, 2, 2, 3, true>(a, st);
    const int64_t tall8 = ((a.N + 127) / 128) * ((a.T + 255) / 256);
    if (4 * tall8 >= 3 * ncu) return gemm_cfg<128, 256, 128, 2, 4, 2, true>(a, st);
    const int64_t mid8 = ((a.N + 127) / 128) * ((a.T + 127) / 128);
    if (mid8 >= ncu) return gemm_cfg<128, 128, 256, 2, 2, 2, true>(a, st);
    return gemm_cfg<64, 64, 256, 2, 2, 2, true>(a, st);
  }
  // 256x256 tiles when they fill the chip at least once; the big tile runs 16
  // waves of 64x64 (4 per SIMD): with fewer, larger wave tiles the per-stage
  // barrier and LDS latency are not covered (measured ~8% slower).  Smaller
  // problems are latency-bound: 128x128 tiles, else 64x64 tiles (two workgroups
  // per CU), both with two 256-byte K stages, which halve the stage count
  // against 128-byte stages in a 4-deep ring of the same LDS size:
  // 512x4096x4096 17.7 us, 1024x4096x4096 26.3 us and 128x1024x1024 5.2 us,
  // against 19.1, 28.3 and 5.6 us.
  // More 256x256 tiles than CUs: the persistent form (one workgroup per CU
  // walks its tiles and streams the next tile's first stage during the
  // epilogue; measured 2-3% faster on 8192^3 and 2048x16384x4096).
  const int64_t big = ((a.N + 255) / 256) * ((a.T + 255) / 256);
  if (big >= ncu) return gemm_cfg<256, 256, 128, 4, 4, 2, false, true>(a, st, ncu);
  // At least 3/4 of a 256x256 tile per CU: the big tile still, one per workgroup;
  // its operand reuse outweighs the idle CUs (768x16384x4096 64.0 against 82.9 us,
  // 512x28672x8192 142 against 212 us with 128x128 tiles; at half the CUs it
  // loses: 384x16384x8192 102.8 against 93.4 us).
  if (4 * big >= 3 * ncu) return gemm_cfg<256, 256, 128, 4, 4, 2>(a, st);
  // Up to 128 tokens with many output channels (a batch of decode steps through
  // a wide layer): one 128-token tile per 128 channels (when those fill 3/4 of
  // the CUs), else per 64 channels (three 128-byte stages), reads every weight
  // tile once, where 64x64 tiles read it once per 64 tokens.  With weights
  // streamed from HBM: 96x28672x8192 57.6 (128x128) / 61.2 (64x128) against 69
  // us, 128x14336x4096 20.7 (64x128) against 24.4 us; with fewer channel tiles
  // than 3/4 of the CUs 64x64 tiles stay ahead (8192 channels: 30.7 against 31.3 us).
  if (a.T <= 128 && (a.N + 127) / 128 >= (3 * ncu) / 4) return gemm_cfg<128, 128, 256, 2, 2, 2>(a, st);
  if (a.T <= 128 && (a.N + 63) / 64 >= (3 * ncu) / 4) return gemm_cfg<64, 128, 128, 2, 2, 3>(a, st);
  // Else 128 channels x 256 tokens (8 waves of 64x64, two 128-byte stages) when
  // those tiles fill 3/4 of the CUs: fewer weight re-reads than 128x128 tiles
  // (200x24576x4096 42.1 against 52.8 us, 512x14336x4096 43.0 against 52.5 us,
  // 129-256 x 28672 x 8192 79-87 against 100-115 us; at half the CUs it loses:
  // 160x16384x4096 39.2 against 28.8 us).
  const int64_t tall = ((a.N + 127) / 128) * ((a.T + 255) / 256);
  if (4 * tall >= 3 * ncu) return gemm_cfg<128, 256, 128, 2, 4, 2>(a, st);
  const int64_t mid = ((a.N + 127) / 128) * ((a.T + 127) / 128);
  if (mid >= ncu) return gemm_cfg<128, 128, 256, 2, 2, 2>(a, st);
  return gemm_cfg<64, 64, 256, 2, 2, 2>(a, st);
}

// ---------------------------------------------------------------- generic path
template <int OUT>
__global__ __launch_bounds__(256) void gemm_generic_kernel(const int8_t* __restrict__ Xq,
                                                           const float* __restrict__ xs,
                                                           const int8_t* __restrict__ Wq,
                                                           const float* __restrict__ ws, int64_t T,
                                                           int64_t N, int64_t K, void* __restrict__ Y,
                                                           const float* __restrict__ xo,
                                                           const float* __restrict__ wo, int64_t n_o) {
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
      float v = (float)acc * (xs[t] * ws[n]);
      if (n_o > 0) {
        float so = 0.0f;
        for (int64_t q = 0; q < n_o; ++q) so = so + xo[q * T + t] * wo[q * N + n];
        v = v + so;
      }
      if (OUT == kOutF32) static_cast<float*>(Y)[o] = v;
      else static_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_bf16(v);
    }
  }
}

// FP8 codes, any shape and alignment: binary32 sum over k of the decoded
// products, then y = fl32(acc * fl32(xs * ws)).
template <int OUT>
__global__ __launch_bounds__(256) void gemm_fp8_generic_kernel(const uint8_t* __restrict__ Xq,
                                                               const float* __restrict__ xs,
                                                               const uint8_t* __restrict__ Wq,
                                                               const float* __restrict__ ws, int64_t T,
                                                               int64_t N, int64_t K, void* __restrict__ Y) {
  const int64_t total = T * N;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < total;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int64_t t = o / N, n = o - t * N;
    const uint8_t* x = Xq + t * K;
    const uint8_t* w = Wq + n * K;
    float acc = 0.0f;
    for (int64_t k = 0; k < K; ++k) acc = acc + e4m3_value(x[k]) * e4m3_value(w[k]);
    const float v = acc * (xs[t] * ws[n]);
    if (OUT == kOutF32) static_cast<float*>(Y)[o] = v;
    else static_cast<uint16_t*>(Y)[o] = (uint16_t)f32_to_bf16(v);
  }
}

hipError_t launch_gemm_generic(const GemmArgs& a, hipStream_t st) {
  if (a.f8) {
    int64_t g = (a.T * a.N + 255) / 256;
    if (g > 65536) g = 65536;
    SQ_TRACE("gemm_fp8_generic (scalar; K %% 16 != 0 or unaligned operands) T %lld N %lld K %lld, grid %lld x 256 threads",
             (long long)a.T, (long long)a.N, (long long)a.K, (long long)g);
    const uint8_t* xq = reinterpret_cast<const uint8_t*>(a.Xq);
    const uint8_t* wq = reinterpret_cast<const uint8_t*>(a.Wq);
    if (a.out == kOutF32)
      hipLaunchKernelGGL(gemm_fp8_generic_kernel<kOutF32>, dim3((unsigned)g), dim3(256), 0, st, xq, a.xs, wq, a.ws, a.T, a.N, a.K, a.Y);
    else
      hipLaunchKernelGGL(gemm_fp8_generic_kernel<kOutBF16>, dim3((unsigned)g), dim3(256), 0, st, xq, a.xs, wq, a.ws, a.T, a.N, a.K, a.Y);
    return hipGetLastError();
  }
  int64_t total = a.T * a.N;
  int64_t g = (total + 255) / 256;
  if (g > 65536) g = 65536;
  dim3 grid((unsigned)g), block(256);
  SQ_TRACE("gemm_generic (scalar; K %% 16 != 0 or unaligned operands) T %lld N %lld K %lld, grid %lld x 256 threads",
           (long long)a.T, (long long)a.N, (long long)a.K, (long long)g);
  switch (a.out) {
    case kOutF32:
      hipLaunchKernelGGL(gemm_generic_kernel<kOutF32>, grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y,
                         a.xo, a.wo, a.out == kOutI32 ? 0 : a.n_o);
      break;
    case kOutBF16:
      hipLaunchKernelGGL(gemm_generic_kernel<kOutBF16>, grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y,
                         a.xo, a.wo, a.out == kOutI32 ? 0 : a.n_o);
      break;
    default:
      hipLaunchKernelGGL(gemm_generic_kernel<kOutI32>, grid, block, 0, st, a.Xq, a.xs, a.Wq, a.ws, a.T, a.N, a.K, a.Y,
                         a.xo, a.wo, a.out == kOutI32 ? 0 : a.n_o);
      break;
  }
  return hipGetLastError();
}

}  // namespace sq
