// Integer GEMM of libhq for gfx950: int8 codes (int4 codes ride in int8
// lanes losslessly), v_mfma_i32_32x32x32_i8 with int32 accumulation
// (HaTQ Sec. III-B Eq. (4), zero points 0), and a fused epilogue
//   Y = acc * s_x[m] * s_w[n] + b[n] + mu[m] * c[n]  [+ U[m,:] . L2[:, n]]
// (HaTQ Eq. (18) accumulator scale; HadaNorm Eq. (1) bias correction; the
// low-rank term of the data-free int4 blog, step 4, on bf16 MFMA).
//
// Operands: A [M, K] (activation codes, K contiguous), B [N, K] (weight
// codes, K contiguous): a "TN" product, so each lane feeds 16 consecutive
// bytes of one row to the MFMA without any transposition.
//
// Tiling: BM x BN macro tile per 256-thread block, BK = 128 bytes of K per
// stage, double-buffered in LDS. Rows of a stage tile are 128 B (8 chunks of
// 16 B); chunk c of row r is stored at slot c ^ (r & 7), so the 32 lanes that
// read one 16-B chunk column from 32 consecutive rows hit distinct banks.
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {

constexpr int BK = 128;

__device__ __forceinline__ int swz(int row, int chunk) { return (row << 7) + ((chunk ^ (row & 7)) << 4); }

// s_waitcnt with vmcnt = N (vector-memory ops still allowed in flight) and
// lgkmcnt = 0 (every LDS read issued by this wave has returned).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

__device__ __forceinline__ v8bf pack_bf16x8(const float f[8], bool residual) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint16_t h0 = f32_to_bf16(f[2 * q]), h1 = f32_to_bf16(f[2 * q + 1]);
    if (residual) {
      h0 = f32_to_bf16(f[2 * q] - bf16_to_f32(h0));
      h1 = f32_to_bf16(f[2 * q + 1] - bf16_to_f32(h1));
    }
    w[q] = uint32_t(h0) | (uint32_t(h1) << 16);
  }
  return __builtin_bit_cast(v8bf, make_uint4(w[0], w[1], w[2], w[3]));
}

// Stage loads go straight from global memory to LDS (gfx950
// global_load_lds_dwordx4): one instruction moves 64 lanes x 16 B into 1 KB of
// consecutive LDS, lane l landing in slot l. The lane therefore fetches the
// global chunk that belongs in that swizzled slot. Waits and barriers are
// explicit (bare s_barrier): stage kt+S-1 is issued right after the barrier
// that retires stage kt-1, so S-1 stages are in flight behind the MFMAs.
template <int BM, int BN, int WM, int WN, int S, bool DEQ>
__global__ __launch_bounds__(256) void gemm_i8_kernel(
    const int8_t* __restrict__ A, int64_t M, const int8_t* __restrict__ B, int64_t N, int K,
    int32_t* __restrict__ Cout, int64_t ldc, GemmEpi ep) {
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int WAVES_N = BN / WN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int LA = BM / (8 * NW), LB = BN / (8 * NW), L = LA + LB;
  static_assert(LA * 8 * NW == BM && LB * 8 * NW == BN, "whole load instructions per wave");
  static_assert(S >= 2 && S <= 4, "2..4 stages");
  constexpr int STAGE = (BM + BN) * BK;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t m0 = int64_t(blockIdx.y) * BM, n0 = int64_t(blockIdx.x) * BN;
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;
  const int KT = K / BK;

  // Per load instruction q: global row pointer (rows clamped into range) and
  // the 1-KB LDS block it fills.
  const int8_t* gsrc[L];
  int ldst[L];
#pragma unroll
  for (int q = 0; q < L; ++q) {
    const bool isA = q < LA;
    const int blk = (isA ? q : q - LA) * NW + wave;   // 1-KB block index in the A or B tile
    const int slot = blk * 64 + lane;                 // 16-B slot index
    const int row = slot >> 3, c = (slot & 7) ^ (row & 7);
    int64_t gr = (isA ? m0 : n0) + row;
    const int64_t lim = (isA ? M : N) - 1;
    if (gr > lim) gr = lim;
    gsrc[q] = (isA ? A : B) + gr * K + c * 16;
    ldst[q] = (isA ? 0 : BM * BK) + blk * 1024;
  }
#define HQ_ISSUE_STAGE(KT_)                                                              \
  do {                                                                                   \
    uint8_t* base_ = smem + ((KT_) % S) * STAGE;                                         \
    _Pragma("unroll") for (int q = 0; q < L; ++q)                                        \
        lds_dma16(gsrc[q] + (KT_) * BK, base_ + ldst[q]);                                \
  } while (0)

  v16i acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v16i{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

#pragma unroll
  for (int p = 0; p < S - 1; ++p)
    if (p < KT) HQ_ISSUE_STAGE(p);

  const int lrow = lane & 31, lhalf = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    // Stage kt must have landed; up to min(S-2, KT-1-kt) later stages may fly.
    const int ahead = KT - 1 - kt;
    if (S >= 4 && ahead >= 2)
      wait_vm_lgkm0<(S >= 4 ? 2 * L : 0)>();
    else if (S >= 3 && ahead >= 1)
      wait_vm_lgkm0<(S >= 3 ? L : 0)>();
    else
      wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    if (kt + S - 1 < KT) HQ_ISSUE_STAGE(kt + S - 1);

    const uint8_t* cur = smem + (kt % S) * STAGE;
#pragma unroll
    for (int s = 0; s < BK / 32; ++s) {
      const int c = 2 * s + lhalf;
      v4i af[TM], bfr[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const v4i*>(cur + swz(wm0 + i * 32 + lrow, c));
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfr[j] = *reinterpret_cast<const v4i*>(cur + BM * BK + swz(wn0 + j * 32 + lrow, c));
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
  }

  // 32x32 accumulator layout: lane l, register r ->
  //   column (l % 32), row 8*(r/4) + 4*(l/32) + (r % 4).
  if constexpr (!DEQ) {
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn0 + j * 32 + lrow;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm0 + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
          if (m < M && n < N) Cout[m * ldc + n] = acc[i][j][r];
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      float sx[16], mu[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        int64_t m = m0 + wm0 + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
        if (m > M - 1) m = M - 1;
        sx[r] = ep.s_x[m];
        mu[r] = ep.mu[m];
      }
      // Low-rank rows of this 32-row strip: lane supplies row (l % 32).
      int64_t um = m0 + wm0 + i * 32 + lrow;
      if (um > M - 1) um = M - 1;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t n = n0 + wn0 + j * 32 + lrow;
        const int64_t nc = n < N ? n : N - 1;
        const float sw = ep.s_w[nc], cb = ep.c[nc], bb = ep.bias[nc];
        v16f lr = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        for (int k0 = 0; k0 < ep.rank; k0 += 16) {
          float f[8];
          load8(ep.U + um * ep.rank + k0 + 8 * lhalf, f);
          const v8bf uh = pack_bf16x8(f, false), ul = pack_bf16x8(f, true);
          const int64_t off = nc * ep.rank + k0 + 8 * lhalf;
          const v8bf wh = *reinterpret_cast<const v8bf*>(ep.l2_hi + off);
          const v8bf wl = *reinterpret_cast<const v8bf*>(ep.l2_lo + off);
          lr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uh, wh, lr, 0, 0, 0);
          lr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(uh, wl, lr, 0, 0, 0);
          lr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ul, wh, lr, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + wm0 + i * 32 + 8 * (r >> 2) + 4 * lhalf + (r & 3);
          const float y = float(acc[i][j][r]) * (sx[r] * sw) + (bb + mu[r] * cb) + lr[r];
          if (m < M && n < N) {
            if (ep.y_bf16)
              static_cast<uint16_t*>(ep.Y)[m * ep.ldy + n] = f32_to_bf16(y);
            else
              static_cast<float*>(ep.Y)[m * ep.ldy + n] = y;
          }
        }
      }
    }
  }
}

hipError_t launch_gemm(const int8_t* A, int64_t M, const int8_t* B, int64_t N, int K,
                       int32_t* acc_out, int64_t ldc, const GemmEpi* epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % BK) return hipErrorInvalidValue;
  constexpr int BM = 128, BN = 128, WM = 64, WN = 64, S = 3;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  dim3 grid{unsigned((N + BN - 1) / BN), unsigned((M + BM - 1) / BM)}, block{NT};
  GemmEpi ep = {};
  if (epi) {
    ep = *epi;
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM, WN, S, true>), grid, block, 0, s, A, M, B, N,
                       K, nullptr, 0, ep);
  } else {
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, WM, WN, S, false>), grid, block, 0, s, A, M, B, N,
                       K, acc_out, ldc, ep);
  }
  return hipGetLastError();
}

}  // namespace hq
