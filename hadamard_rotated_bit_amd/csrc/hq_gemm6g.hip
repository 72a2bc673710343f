// Group-wise FP6 (E2M3) GEMM of libhq: 4-bit codes with one scale per row and
// 64-channel group on both sides (data-free int4 blog, "Hadamard rotation:
// the int4 improvement": every group of 64 input channels shares one scale,
// and the rotation uses one 64 x 64 Hadamard block per group):
//
//   Y_tj = sum_g s_x[g, t] s_w[g, j] (sum_{k in g} qa_tk qw_jk) + b_j + mu_t c_j (+ U L2)
//
// The codes use the common E2M3 layout (hq_gemm6_kernel.h). A 128-code stage
// holds two groups. Where the per-row kernel pairs codes 0-31 with 64-95 in
// one MFMA, here lane half h reads the 24-byte pieces [24h, 24h+24) and
// [48+24h, 72+24h) of each 96-byte row segment, so the first
// v_mfma_f32_32x32x64_f8f6f4 of a stage takes codes 0-63 (group 2 kt) and the
// second codes 64-127 (group 2 kt + 1). Each MFMA writes a zeroed temporary;
// its 16 values per lane are added to the accumulators scaled by
// s_x[g, row] s_w[g, col] (fp32 VALU; exact integers times the scales).
//
// Tiles 128 x 128, 4 waves of 64 x 64. Stage buffer = A and B codes plus the
// stage's four scale vectors (s_x and s_w of both groups), all by
// buffer_load ... lds against per-tile descriptors (rows past M / N and stages
// past K move nothing). With S buffers, iteration kt waits for stage kt
// (S = 3: stage kt+1 may stay in flight), joins the block (every wave is done
// with stage kt-1), refills stage kt-1's buffer with stage kt+S-1, then reads
// stage kt's fragments and scales and runs its two groups. The launch uses
// S = 2 and three blocks per CU (168 VGPRs, 3 x 53 KB of LDS): the rescale
// keeps the VALU busy, and three independent blocks per SIMD hide each
// other's loads, barriers and epilogues better than two blocks with a deeper
// pipeline (measured on flux_g64: 242 vs 303 us).
#include "hq_gemm6_kernel.h"
#include "hq_internal.h"

namespace hq {

// A fragment from its six 8-byte pieces (two 24-byte operands).
__device__ __forceinline__ void frag_from_pieces(Frag6& f, const v2i* q) {
  f.c[0] = v4i{q[0].x, q[0].y, q[1].x, q[1].y};
  f.c[1] = v4i{q[2].x, q[2].y, q[3].x, q[3].y};
  f.c[2] = v4i{q[4].x, q[4].y, q[5].x, q[5].y};
}

// MFMA of tile n of a stage (two groups, TM x TN 32 x 32 tiles per group):
// group n / (TM TN), column strip (n / TM) % TN, row strip n % TM, into a
// zeroed temporary.
template <int TM, int TN, int N>
__device__ __forceinline__ v16f group_tile_mfma(const Frag6 (&af)[TM], const Frag6 (&bf)[TN]) {
  constexpr int g = N / (TM * TN), j = (N / TM) % TN, i = N % TM;
  const v16f zero = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  if constexpr (g == 0) return mfma_f6(f6_op0(bf[j]), f6_op0(af[i]), zero);
  else return mfma_f6(f6_op1(bf[j]), f6_op1(af[i]), zero);
}

// Accumulator register r of a lane in half h holds column 8 (r / 4) + 4 h + r % 4
// of its 32-column strip. Lane l holds the scale of column
// 8 ((l % 16) / 4) + 4 (l / 32) + l % 4: the 16 lanes of a row hold the 16
// columns of their half, lane r of the row the one of register r, so DPP
// row_newbcast:r (every lane of a 16-lane row reads lane r of that row) hands
// each lane its register-r scale inside the multiply. Written as one asm
// block (the compiler does not fold the broadcast into a multiply whose
// operand is shared); the leading s_nop covers the two wait states a DPP
// read needs after a VALU write of its source.
__device__ __forceinline__ void scale_products(float (&p)[16], float sw, float sx) {
  asm volatile(
      "s_nop 1\n"
      "v_mul_f32_dpp %0, %16, %17 row_newbcast:0 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %1, %16, %17 row_newbcast:1 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %2, %16, %17 row_newbcast:2 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %3, %16, %17 row_newbcast:3 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %4, %16, %17 row_newbcast:4 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %5, %16, %17 row_newbcast:5 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %6, %16, %17 row_newbcast:6 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %7, %16, %17 row_newbcast:7 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %8, %16, %17 row_newbcast:8 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %9, %16, %17 row_newbcast:9 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %10, %16, %17 row_newbcast:10 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %11, %16, %17 row_newbcast:11 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %12, %16, %17 row_newbcast:12 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %13, %16, %17 row_newbcast:13 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %14, %16, %17 row_newbcast:14 row_mask:0xf bank_mask:0xf\n"
      "v_mul_f32_dpp %15, %16, %17 row_newbcast:15 row_mask:0xf bank_mask:0xf"
      : "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3]), "=&v"(p[4]), "=&v"(p[5]),
        "=&v"(p[6]), "=&v"(p[7]), "=&v"(p[8]), "=&v"(p[9]), "=&v"(p[10]), "=&v"(p[11]),
        "=&v"(p[12]), "=&v"(p[13]), "=&v"(p[14]), "=&v"(p[15])
      : "v"(sw), "v"(sx));
}

// The MFMAs and rescales of one stage: per tile, the MFMA, the tile's 16
// scale products (independent of it, so they issue while it runs), then
// acc += t * s_x * s_w.
template <int TM, int TN, int N, bool PIN>
__device__ __forceinline__ void group_tiles(v16f (&acc)[TM][TN], const Frag6 (&af)[TM],
                                           const Frag6 (&bf)[TN], const float (&sx)[2][TM],
                                           const float (&sw)[2][TN]) {
  if constexpr (N < 2 * TM * TN) {
    constexpr int g = N / (TM * TN), j = (N / TM) % TN, i = N % TM;
    const v16f t = group_tile_mfma<TM, TN, N>(af, bf);
    float p[16];
    scale_products(p, sw[g][j], sx[g][i]);
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][j][r] = fmaf(t[r], p[r], acc[i][j][r]);
    if constexpr (PIN) __builtin_amdgcn_sched_barrier(0);
    group_tiles<TM, TN, N + 1, PIN>(acc, af, bf, sx, sw);
  }
}

template <int BM, int BN, int WM, int WN, int GM, int RG, int S = 3, int OCC = 2>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(OCC))) void gemm_f6g_kernel(
    const uint8_t* __restrict__ A, int64_t M, const uint8_t* __restrict__ B, int64_t N, int K,
    GemmEpi ep, const float* __restrict__ sxg, int64_t ldsx, const float* __restrict__ swg,
    int64_t ldsw) {
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int WAVES_N = BN / WN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int CODEB = 96 * (BM + BN);
  constexpr int STAGE = CODEB + 8 * (BM + BN);  // + two groups of row and column scales
  constexpr int UA = 3 * BM / 32;
  constexpr int UNITS = 3 * (BM + BN) / 32;
  constexpr int LPW = UNITS / NW;
  constexpr int QA = UA / NW;
  constexpr int UV = BM / 64;                    // 64-float units per scale vector
  constexpr int SPW = 4 * UV / NW;               // scale units per wave and stage
  static_assert(BM == BN && BM % 64 == 0, "square tiles of whole scale units");
  static_assert(UNITS % NW == 0 && UA % NW == 0 && (4 * UV) % NW == 0, "even DMA split");
  static_assert(S == 2 || S == 3, "two or three stage buffers");
  static_assert(BM * (2 * BN + 8) + 4 * (3 * BN + 2 * BM) <= S * STAGE,
                "epilogue tile and parameters fit in the stage buffers");
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  int64_t m0, n0;
  f6_tile_origin<BM, BN, GM>(int(blockIdx.x), M, N, &m0, &n0);
  const int wm0 = (wv / WAVES_N) * WM, wn0 = (wv % WAVES_N) * WN;
  const int KT = K / 128;
  const int64_t lda = f6_row_bytes(K);

  const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
  const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
  const uint8_t* abase = A + m0 * lda;
  const uint8_t* bbase = B + n0 * lda;
  const int nrec_a = int((rows_a + RG - 1) / RG * RG * lda);
  const int nrec_b = int((rows_b + RG - 1) / RG * RG * lda);
  uint32_t voff[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    const int u = q * NW + wv;
    const int ul = q < QA ? u : u - UA;
    const int c = 64 * ul + lane;
    const int row = c / 6, slot = c - 6 * (c / 6);
    const int h = (slot >= 3 ? 1 : 0) ^ ((row >> 3) & 1);
    voff[q] = uint32_t((row / RG) * RG * lda + (row % RG) * 96 + 48 * h +
                       16 * (slot - 3 * (slot >= 3 ? 1 : 0)));
  }

  // Stage KT_ into buffer BUF_: codes, then the scale vectors
  // [s_x g0 | s_x g1 | s_w g0 | s_w g1] (BM floats each; 64-float units).
#define HG_ISSUE(KT_, BUF_)                                                                \
  do {                                                                                     \
    const int kt_ = (KT_);                                                                 \
    uint8_t* base_ = smem + (BUF_) * STAGE;                                                \
    const bool ok_ = kt_ < KT;                                                             \
    const __amdgpu_buffer_rsrc_t ra_ = make_rsrc(abase, ok_ ? nrec_a : 0);                 \
    const __amdgpu_buffer_rsrc_t rb_ = make_rsrc(bbase, ok_ ? nrec_b : 0);                 \
    _Pragma("unroll") for (int q = 0; q < LPW; ++q)                                        \
        lds_dma16_buf(q < QA ? ra_ : rb_, voff[q], uint32_t(kt_) * (96u * RG),             \
                      base_ + (q * NW + wv) * 1024);                                       \
    _Pragma("unroll") for (int q = 0; q < SPW; ++q) {                                      \
      const int u_ = q * NW + wv, vec_ = u_ / UV, part_ = u_ - vec_ * UV;                  \
      const bool colv_ = vec_ >= 2;                                                        \
      const int64_t g_ = 2 * int64_t(kt_) + (vec_ & 1);                                    \
      const int64_t first_ = (colv_ ? n0 : m0) + 64 * part_;                               \
      const int64_t lim_ = (colv_ ? N : M) - first_;                                       \
      const float* src_ = colv_ ? swg + g_ * ldsw + first_ : sxg + g_ * ldsx + first_;     \
      const int nb_ = ok_ ? int((lim_ < 64 ? (lim_ > 0 ? lim_ : 0) : 64) * 4) : 0;         \
      lds_dma4_buf(make_rsrc(src_, nb_), uint32_t(lane) * 4u, 0u,                          \
                   base_ + CODEB + vec_ * 4 * BM + part_ * 256);                           \
    }                                                                                      \
  } while (0)

  // Fragment of a row: dwords 0-5 = logical bytes [24h, 24h+24) (group 0),
  // dwords 6-11 = [48+24h, 72+24h) (group 1); rows with bit 3 set hold their
  // 48-byte halves swapped. Scales: s_x of the lane's rows wm0 + lrow +
  // {0, 32}; s_w of column 8 ((l % 16) / 4) + 4 (l / 32) + l % 4 of each
  // 32-column strip (see scale_products). The LDS reads are written as inline asm that
  // waits for its own results: the compiler would otherwise wait for every
  // stage load in flight (it cannot tell that they fill other buffers).
  static_assert(TM == 2 && TN == 2, "fragment reads are written for 64 x 64 waves");
  const int lrow = lane & 31, lhalf = lane >> 5;
  const int swp = ((lrow >> 3) & 1) * 48;
  const uint32_t lds0 = uint32_t(reinterpret_cast<uintptr_t>(smem));
  const uint32_t pa0 = lds0 + uint32_t(wm0 * 96 + lrow * 96 + (24 * lhalf + swp) % 96);
  const uint32_t pa1 = lds0 + uint32_t(wm0 * 96 + lrow * 96 + (48 + 24 * lhalf + swp) % 96);
  const uint32_t pb0 = pa0 + uint32_t((BM + wn0 - wm0) * 96);
  const uint32_t pb1 = pa1 + uint32_t((BM + wn0 - wm0) * 96);
  const uint32_t psx = lds0 + uint32_t(CODEB + 4 * (wm0 + lrow));
  const uint32_t psw =
      lds0 + uint32_t(CODEB + 4 * (2 * BM + wn0 + 8 * ((lane & 15) >> 2) + 4 * lhalf + (lane & 3)));
#define HG_READ(BUF_)                                                                      \
  do {                                                                                     \
    const uint32_t o_ = uint32_t(BUF_) * STAGE;                                            \
    v2i r_[24];                                                                            \
    asm volatile(                                                                          \
        "ds_read_b64 %0, %24\n ds_read_b64 %1, %24 offset:8\n ds_read_b64 %2, %24 offset:16\n" \
        "ds_read_b64 %3, %25\n ds_read_b64 %4, %25 offset:8\n ds_read_b64 %5, %25 offset:16\n" \
        "ds_read_b64 %6, %24 offset:3072\n ds_read_b64 %7, %24 offset:3080\n"              \
        "ds_read_b64 %8, %24 offset:3088\n ds_read_b64 %9, %25 offset:3072\n"              \
        "ds_read_b64 %10, %25 offset:3080\n ds_read_b64 %11, %25 offset:3088\n"            \
        "ds_read_b64 %12, %26\n ds_read_b64 %13, %26 offset:8\n ds_read_b64 %14, %26 offset:16\n" \
        "ds_read_b64 %15, %27\n ds_read_b64 %16, %27 offset:8\n ds_read_b64 %17, %27 offset:16\n" \
        "ds_read_b64 %18, %26 offset:3072\n ds_read_b64 %19, %26 offset:3080\n"            \
        "ds_read_b64 %20, %26 offset:3088\n ds_read_b64 %21, %27 offset:3072\n"            \
        "ds_read_b64 %22, %27 offset:3080\n ds_read_b64 %23, %27 offset:3088\n"            \
        "s_waitcnt lgkmcnt(0)"                                                             \
        : "=&v"(r_[0]), "=&v"(r_[1]), "=&v"(r_[2]), "=&v"(r_[3]), "=&v"(r_[4]),            \
          "=&v"(r_[5]), "=&v"(r_[6]), "=&v"(r_[7]), "=&v"(r_[8]), "=&v"(r_[9]),            \
          "=&v"(r_[10]), "=&v"(r_[11]), "=&v"(r_[12]), "=&v"(r_[13]), "=&v"(r_[14]),       \
          "=&v"(r_[15]), "=&v"(r_[16]), "=&v"(r_[17]), "=&v"(r_[18]), "=&v"(r_[19]),       \
          "=&v"(r_[20]), "=&v"(r_[21]), "=&v"(r_[22]), "=&v"(r_[23])                       \
        : "v"(pa0 + o_), "v"(pa1 + o_), "v"(pb0 + o_), "v"(pb1 + o_)                       \
        : "memory");                                                                       \
    frag_from_pieces(af[0], r_ + 0);                                                       \
    frag_from_pieces(af[1], r_ + 6);                                                       \
    frag_from_pieces(bf[0], r_ + 12);                                                      \
    frag_from_pieces(bf[1], r_ + 18);                                                      \
  } while (0)
  // Both groups of the stage in buffer BUF_: MFMA into a zeroed temporary,
  // then acc += temp * s_x[row] * s_w[col]. Group GI_'s scales: s_x of the
  // lane's rows wm0 + lrow + {0, 32}, s_w of its 16 columns.
#define HG_SCALES(BUF_)                                                                    \
  do {                                                                                     \
    const uint32_t o_ = uint32_t(BUF_) * STAGE;                                            \
    asm volatile(                                                                          \
        "ds_read_b32 %0, %8\n ds_read_b32 %1, %8 offset:128\n"                            \
        "ds_read_b32 %2, %8 offset:512\n ds_read_b32 %3, %8 offset:640\n"                 \
        "ds_read_b32 %4, %9\n ds_read_b32 %5, %9 offset:128\n"                            \
        "ds_read_b32 %6, %9 offset:512\n ds_read_b32 %7, %9 offset:640\n"                 \
        "s_waitcnt lgkmcnt(0)"                                                             \
        : "=&v"(sx_[0][0]), "=&v"(sx_[0][1]), "=&v"(sx_[1][0]), "=&v"(sx_[1][1]),          \
          "=&v"(sw_[0][0]), "=&v"(sw_[0][1]), "=&v"(sw_[1][0]), "=&v"(sw_[1][1])           \
        : "v"(psx + o_), "v"(psw + o_)                                                     \
        : "memory");                                                                       \
  } while (0)
#define HG_MATH(BUF_)                                                                      \
  do {                                                                                     \
    float sx_[2][TM];                                                                      \
    float sw_[2][TN];                                                                      \
    HG_SCALES(BUF_);                                                                       \
    group_tiles<TM, TN, 0, (OCC > 2)>(acc, af, bf, sx_, sw_);                              \
  } while (0)
#define HG_STEP(KT_)                                                                       \
  do {                                                                                     \
    wait_vm_lgkm0<(S - 2) * (LPW + SPW)>();                                                \
    __builtin_amdgcn_s_barrier();                                                          \
    const int cb_ = (KT_) % S;                                                             \
    HG_ISSUE((KT_) + S - 1, cb_ == 0 ? S - 1 : cb_ - 1);                                   \
    HG_READ(cb_);                                                                          \
    HG_MATH(cb_);                                                                          \
  } while (0)

  const v16f zero = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = zero;
  Frag6 af[TM], bf[TN];

  HG_ISSUE(0, 0);
  if constexpr (S == 3) HG_ISSUE(1, 1);
  for (int kt = 0; kt < KT; ++kt) HG_STEP(kt);
  wait_vm_lgkm0<0>();   // no LDS write may land after the block ends
#undef HG_STEP
#undef HG_MATH
#undef HG_SCALES
#undef HG_SCALES
#undef HG_READ
#undef HG_ISSUE

  if (ep.y_bf16) {
    // bf16 output staged through LDS (whole row segments per store). The
    // accumulators already carry both scales, so the staged parameter block
    // holds unit s_w and s_x next to c, b and mu, right after the output tile.
    float* P = reinterpret_cast<float*>(smem + BM * (2 * BN + 8));
    __builtin_amdgcn_s_barrier();   // every wave is past its last stage read
    for (int idx = tid; idx < BN; idx += NW * 64) {
      const int64_t nc = n0 + idx < N ? n0 + idx : N - 1;
      P[idx] = 1.0f;
      P[BN + idx] = ep.c[nc];
      P[2 * BN + idx] = ep.bias[nc];
    }
    for (int idx = tid; idx < BM; idx += NW * 64) {
      const int64_t mc = m0 + idx < M ? m0 + idx : M - 1;
      P[3 * BN + idx] = 1.0f;
      P[3 * BN + BM + idx] = ep.mu[mc];
    }
    __syncthreads();
    if (ep.rank)
      gemm_epilogue_bf16_staged<BM, BN, TM, TN, NW, true>(acc, smem, P, tid, lane, m0, n0, wm0,
                                                          wn0, M, N, ep);
    else
      gemm_epilogue_bf16_staged<BM, BN, TM, TN, NW, false>(acc, smem, P, tid, lane, m0, n0, wm0,
                                                           wn0, M, N, ep);
    return;
  }
  gemm_epilogue<BM, BN, TM, TN, NW, true>(acc, smem, tid, lane, m0, n0, wm0, wn0, M, N, nullptr,
                                         0, ep);
}

hipError_t launch_gemm_f6g(const uint8_t* A, int64_t M, const uint8_t* B, int64_t N, int K,
                           const float* s_xg, int64_t ld_sx, const float* s_wg, int64_t ld_sw,
                           const GemmEpi* epi, hipStream_t s) {
  if (M <= 0 || N <= 0) return hipSuccess;
  if (K % 128 || K > 8192 || !epi) return hipErrorInvalidValue;
  constexpr int BM = 128, BN = 128;
  const int64_t ntiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  GemmEpi ep = *epi;
  ep.prescaled = 1;
  hipLaunchKernelGGL((gemm_f6g_kernel<BM, BN, 64, 64, 4, F6_GROUP, 2, 3>), dim3(unsigned(ntiles)),
                     dim3(256), 0, s, A, M, B, N, K, ep, s_xg, ld_sx, s_wg, ld_sw);
  return hipGetLastError();
}

}  // namespace hq
