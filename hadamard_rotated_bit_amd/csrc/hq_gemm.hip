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
// Kernel structure (tiles, LDS swizzle, direct-to-LDS staging, XCD-aware tile
// order) is described in hq_gemm_kernel.h. Three tile shapes are used:
//   256 x 256 (8 waves, 128 x 64 each)  large problems;
//   128 x 192 (4 waves, 2 blocks / CU)  K <= 2048 with d_out % 192 == 0, where
//                                       the 192-wide tiles fill whole waves of CUs;
//   128 x 128 (4 waves)                 narrow outputs (d_out <= 512).
// bf16 outputs of larger problems take the persistent kernel instead
// (gemm_i8_persist, hq_gemm6_kernel.h: one block per CU walking 256 x 192
// tiles with the stage pipeline running across tile boundaries).
#include "hq_gemm6_kernel.h"
#include "hq_internal.h"

namespace hq {

template <int BM, int BN, int BK, int WM, int WN, int S, int GM, int OCC>
static hipError_t launch_cfg(const int8_t* A, int64_t M, const int8_t* B, int64_t N, int K,
                             int32_t* acc_out, int64_t ldc, const GemmEpi* epi, hipStream_t s) {
  if (K % BK) return hipErrorInvalidValue;
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const int64_t ntiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid{unsigned(ntiles)}, block{NT};
  GemmEpi ep = {};
  if (epi) {
    ep = *epi;
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, S, GM, true, OCC>), grid, block, 0, s,
                       A, M, B, N, K, nullptr, 0, ep);
  } else {
    hipLaunchKernelGGL((gemm_i8_kernel<BM, BN, BK, WM, WN, S, GM, false, OCC>), grid, block, 0, s,
                       A, M, B, N, K, acc_out, ldc, ep);
  }
  return hipGetLastError();
}

template <int LR>
static hipError_t launch_i8_persist(const int8_t* A, int64_t M, const int8_t* B, int64_t N, int K,
                                    const GemmEpi& ep, int cus, hipStream_t s) {
  const int64_t ntiles = ((M + 255) / 256) * ((N + 191) / 192);
  const unsigned grid = unsigned(ntiles < cus ? ntiles : cus);
  hipLaunchKernelGGL((gemm_i8_persist<256, 192, 128, 96, 4, LR>), dim3(grid), dim3(256), 0, s,
                     reinterpret_cast<const uint8_t*>(A), M, reinterpret_cast<const uint8_t*>(B),
                     N, K, ep);
  return hipGetLastError();
}

static int cu_count() {
  // CU count per device, queried once (racing writers store the same value).
  static int cu_cache[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cu_cache[dev] <= 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
      cu_cache[dev] = n;
  }
  return cu_cache[dev] > 0 ? cu_cache[dev] : 256;
}

hipError_t launch_gemm(const int8_t* A, int64_t M, const int8_t* B, int64_t N, int K,
                       int32_t* acc_out, int64_t ldc, const GemmEpi* epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (epi && epi->y_bf16 && K % 64 == 0 && K >= 256 && M > 512 && N > 512) {
    const int cus = cu_count();
    return !epi->rank         ? launch_i8_persist<0>(A, M, B, N, K, *epi, cus, s)
           : epi->l2_lo_zero ? launch_i8_persist<1>(A, M, B, N, K, *epi, cus, s)
                             : launch_i8_persist<2>(A, M, B, N, K, *epi, cus, s);
  }
  if (N <= 512 || M <= 512)
    return launch_cfg<128, 128, 128, 64, 64, 3, 8, 1>(A, M, B, N, K, acc_out, ldc, epi, s);
  if (K <= 2048 && N % 192 == 0)
    return launch_cfg<128, 192, 128, 64, 96, 2, 8, 2>(A, M, B, N, K, acc_out, ldc, epi, s);
  return launch_cfg<256, 256, 128, 128, 64, 2, 4, 1>(A, M, B, N, K, acc_out, ldc, epi, s);
}

}  // namespace hq
