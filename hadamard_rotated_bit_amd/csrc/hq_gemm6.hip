// FP6 (E2M3) GEMM launcher of libhq for 4-bit codes: the same product and
// epilogue as the int8 path (hq_gemm.hip), on v_mfma_f32_32x32x64_f8f6f4.
// Kernel structure in hq_gemm6_kernel.h.
#include "hq_gemm6_kernel.h"
#include "hq_internal.h"

namespace hq {

template <int BM, int BN, int WM, int WN>
static hipError_t launch_f6_cfg(const uint8_t* A, int64_t M, const uint8_t* B, int64_t N, int K,
                                int32_t* acc_out, int64_t ldc, const GemmEpi* epi, hipStream_t s) {
  constexpr int NT = (BM / WM) * (BN / WN) * 64;
  const int64_t ntiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  dim3 grid{unsigned(ntiles)}, block{NT};
  GemmEpi ep = {};
  if (epi) {
    ep = *epi;
    hipLaunchKernelGGL((gemm_f6_kernel<BM, BN, WM, WN, 3, 4, true, F6_GROUP>), grid, block, 0, s,
                       A, M, B, N, K, nullptr, 0, ep);
  } else {
    hipLaunchKernelGGL((gemm_f6_kernel<BM, BN, WM, WN, 3, 4, false, F6_GROUP>), grid, block, 0, s,
                       A, M, B, N, K, acc_out, ldc, ep);
  }
  return hipGetLastError();
}

// Persistent 256 x 192 kernel for bf16 outputs (K >= 384): one block per CU
// (at most one per tile) walks its tiles with the stage pipeline running
// across tile boundaries.
template <int LR>
static hipError_t launch_f6_persist(const uint8_t* A, int64_t M, const uint8_t* B, int64_t N,
                                    int K, const GemmEpi& ep, int cus, hipStream_t s) {
  const int64_t ntiles = ((M + 255) / 256) * ((N + 191) / 192);
  const unsigned grid = unsigned(ntiles < cus ? ntiles : cus);
  hipLaunchKernelGGL((gemm_f6_persist<256, 192, 128, 96, 4, F6_GROUP, LR>), dim3(grid), dim3(256),
                     0, s, A, M, B, N, K, ep);
  return hipGetLastError();
}

// Tile choice: 256 x 256 or 256 x 192 (one block of 4 waves per CU), whichever
// needs less work per CU once the tiles are dealt in rounds of one per CU
// (rounds x tile width): e.g. 8192 x 4608 takes 3 rounds of 256 x 192 tiles
// instead of 3 rounds of the wider 256 x 256 ones.
hipError_t launch_gemm_f6(const uint8_t* A, int64_t M, const uint8_t* B, int64_t N, int K,
                          int32_t* acc_out, int64_t ldc, const GemmEpi* epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % 128 || K > 8192) return hipErrorInvalidValue;
  // CU count per device, queried once (racing writers store the same value).
  static int cu_cache[64] = {};
  int cus = 256, dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    if (cu_cache[dev] <= 0) {
      int n = 0;
      if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0)
        cu_cache[dev] = n;
    }
    if (cu_cache[dev] > 0) cus = cu_cache[dev];
  }
  if (epi && epi->y_bf16 && K >= 384)
    return !epi->rank         ? launch_f6_persist<0>(A, M, B, N, K, *epi, cus, s)
           : epi->l2_lo_zero ? launch_f6_persist<1>(A, M, B, N, K, *epi, cus, s)
                             : launch_f6_persist<2>(A, M, B, N, K, *epi, cus, s);
  const int64_t tm = (M + 255) / 256;
  const int64_t rounds256 = (tm * ((N + 255) / 256) + cus - 1) / cus;
  const int64_t rounds192 = (tm * ((N + 191) / 192) + cus - 1) / cus;
  if (rounds192 * 192 < rounds256 * 256)
    return launch_f6_cfg<256, 192, 128, 96>(A, M, B, N, K, acc_out, ldc, epi, s);
  return launch_f6_cfg<256, 256, 128, 128>(A, M, B, N, K, acc_out, ldc, epi, s);
}

}  // namespace hq
