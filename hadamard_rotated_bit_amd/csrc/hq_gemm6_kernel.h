// FP6 (E2M3) MFMA GEMM kernel template of libhq for 4-bit codes (gfx950).
//
// Codes in [-7, 7] are exact E2M3 values (e2m3 holds every integer up to 7),
// their products are exact in fp32 and every partial sum stays an integer
// below 2^24 (|acc| <= 49 K with K <= 8192), so
// v_mfma_f32_32x32x64_f8f6f4 with both operands in E2M3 returns the same
// integer dot products as the int8 MFMA (HaTQ Sec. III-B Eq. (4)) at twice
// the dense rate per instruction and 3/4 of the operand bytes.
//
// Code layout (shared by the activation codes and the prepared weights): a
// row of K codes is a little-endian bit string of 6 K bits, code k in bits
// [6k, 6k + 6) as E2M3 (sign bit 5, two exponent bits with bias 1, three
// mantissa bits). Every 128 codes fill 96 bytes (6 chunks of 16 B).
//
// MFMA operands: for one 128-code stage, lane l (row l % 32, half h = l / 32)
// feeds the 48 bytes [48 h, 48 h + 48) of the row as two 24-byte (32-code)
// operands, one per 32x32x64 MFMA. The two MFMAs pair codes 0..31 with
// 64..95 and 32..63 with 96..127 of the stage: every code enters exactly one
// product with its partner at the same K position, since activation and
// weight operands are read with the same map.
//
// LDS: a stage holds the A then the B tile as rows of 96 B in code order,
// except that rows with bit 3 set store their two 48-byte halves swapped.
// A lane reads its 48 bytes as three consecutive ds_read_b128; the 16 lanes
// of one read phase (16 consecutive rows, one half) then start at 16
// distinct 16-B positions of a 256-B bank line (96 r mod 256 repeats every
// 8 rows, the swap moves rows 8..15 by 48 B). Stages are filled by
// buffer_load_dwordx4 ... lds: one instruction writes 1 KB of consecutive LDS
// (64 chunks, about 11 rows) and its lanes fetch whole 96-byte row segments.
//
// Pipeline (S = 3 buffers, one block of 4 waves per CU, 1 wave per SIMD):
// iteration kt waits for stage kt+1 and joins the block, refills the buffer
// of stage kt (its fragments are already in registers) with stage kt+3,
// reads the fragments of stage kt+1 into the second register set and runs
// the MFMAs of stage kt. Each stage load has two iterations to land.
#pragma once

#include "hq_gemm_kernel.h"

namespace hq {

typedef int v8i __attribute__((ext_vector_type(8)));

struct Frag6 {
  v4i c[3];
};

// The 6 dwords of the first / second 32-code operand of a fragment.
__device__ __forceinline__ v8i f6_op0(const Frag6& f) {
  return v8i{f.c[0][0], f.c[0][1], f.c[0][2], f.c[0][3], f.c[1][0], f.c[1][1], 0, 0};
}
__device__ __forceinline__ v8i f6_op1(const Frag6& f) {
  return v8i{f.c[1][2], f.c[1][3], f.c[2][0], f.c[2][1], f.c[2][2], f.c[2][3], 0, 0};
}

// E2M3 x E2M3 -> fp32, 32x32x64 (format code 2 for both operands, no scaling).
__device__ __forceinline__ v16f mfma_f6(const v8i& a, const v8i& b, const v16f& c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 2, 2, 0, 0, 0, 0);
}

// Raw buffer descriptor over `bytes` bytes at `base` (stride 0; gfx9 data
// format word): loads at offsets >= bytes return without touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// 16 bytes per lane from a buffer into LDS (buffer_load_dwordx4 ... lds):
// lane l's bytes land at lds + 16 l.
__device__ __forceinline__ void lds_dma16_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff,
                                              uint32_t soff, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 16, voff, soff, 0, 0);
#endif
}

// Instruction order of one main-loop iteration: NM MFMAs with the NR LDS
// fragment reads spread evenly between them and the NV stage loads spread
// over the first half, so that with one wave per SIMD the reads and loads
// issue while earlier MFMAs execute.
template <int I, int NM, int NR, int NV>
__device__ __forceinline__ void mfma_interleave() {
  if constexpr (I < NM) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    constexpr int r = (I + 1) * NR / NM - I * NR / NM;
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);  // LDS read
    constexpr int H = NM / 2 > 0 ? NM / 2 : 1;
    constexpr int v = I < H ? (I + 1) * NV / H - I * NV / H : 0;
    if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x020, v, 0);  // VMEM read
    mfma_interleave<I + 1, NM, NR, NV>();
  }
}

// 4 bytes per lane from a buffer into LDS (buffer_load_dword ... lds): lane
// l's dword lands at lds + 4 l.
__device__ __forceinline__ void lds_dma4_buf(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                             void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void*)lds, 4, voff, soff, 0, 0);
#endif
}

// Bytes per row of K codes in the fp6 layout.
__host__ __device__ constexpr int64_t f6_row_bytes(int64_t K) { return K / 4 * 3; }

// Origin of tile `tile` of an M x N output in BM x BN tiles: tiles are
// renumbered so that the blocks of one XCD (block b runs on XCD b mod 8) own
// a contiguous range, walked in column-major order inside bands of GM tile
// rows.
template <int BM, int BN, int GM>
__device__ __forceinline__ void f6_tile_origin(int tile, int64_t M, int64_t N, int64_t* m0,
                                               int64_t* n0) {
  const int tmt = int((M + BM - 1) / BM), tnt = int((N + BN - 1) / BN);
  const int ntiles = tmt * tnt;
  if ((ntiles & 7) == 0) tile = (tile & 7) * (ntiles >> 3) + (tile >> 3);
  const int g = tile / (GM * tnt), r = tile - g * (GM * tnt);
  const int rows_in = (tmt - g * GM) < GM ? (tmt - g * GM) : GM;
  *m0 = int64_t(g * GM + r % rows_in) * BM;
  *n0 = int64_t(r / rows_in) * BN;
}

// DMA copy of a tile's epilogue parameters into LDS P = [s_w | c | b] (BN
// each, from column n0) then [s_x | mu] (BM each, from row m0), 64 floats
// (one 4-byte DMA instruction) per unit; entries past N / M are left unread.
// Wave `wv` of NW issues units wv, wv + NW, ... (repeating the last), the
// same count in every wave.
template <int BM, int BN, int NW>
__device__ __forceinline__ void params_dma(uint8_t* P, int wv, int lane, int64_t m0, int64_t n0,
                                           int64_t M, int64_t N, const GemmEpi& ep) {
  constexpr int PU = (3 * BN + 2 * BM) / 64;
  constexpr int PPW = (PU + NW - 1) / NW;
  static_assert(BM % 64 == 0 && BN % 64 == 0, "whole units per vector");
#pragma unroll
  for (int q = 0; q < PPW; ++q) {
    int u = q * NW + wv;
    if (u > PU - 1) u = PU - 1;
    const int f = 64 * u;
    const float* src;
    int64_t lim;
    if (f < BN) {
      src = ep.s_w + n0 + f;
      lim = N - n0 - f;
    } else if (f < 2 * BN) {
      src = ep.c + n0 + (f - BN);
      lim = N - n0 - (f - BN);
    } else if (f < 3 * BN) {
      src = ep.bias + n0 + (f - 2 * BN);
      lim = N - n0 - (f - 2 * BN);
    } else if (f < 3 * BN + BM) {
      src = ep.s_x + m0 + (f - 3 * BN);
      lim = M - m0 - (f - 3 * BN);
    } else {
      src = ep.mu + m0 + (f - 3 * BN - BM);
      lim = M - m0 - (f - 3 * BN - BM);
    }
    const int nrec = int((lim < 64 ? (lim > 0 ? lim : 0) : 64) * 4);
    lds_dma4_buf(make_rsrc(src, nrec), uint32_t(lane) * 4u, 0u, P + 4 * f);
  }
}

template <int BM, int BN, int WM, int WN, int S, int GM, bool DEQ, int RG = 1>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(1))) void gemm_f6_kernel(
    const uint8_t* __restrict__ A, int64_t M, const uint8_t* __restrict__ B, int64_t N, int K,
    int32_t* __restrict__ Cout, int64_t ldc, GemmEpi ep) {
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int WAVES_N = BN / WN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int STAGE = 96 * (BM + BN);
  constexpr int UA = 3 * BM / 32;            // 1-KB DMA units of the A tile
  constexpr int UNITS = 3 * (BM + BN) / 32;
  constexpr int LPW = (UNITS + NW - 1) / NW;  // DMA instructions per wave and stage
  constexpr int QA = UA / NW;                 // the first QA of them load A
  static_assert(UA % NW == 0, "A units split evenly over the waves");
  static_assert(S == 3, "three-buffer pipeline");
  static_assert(BM % 32 == 0 && BN % 32 == 0, "whole 1-KB units per tile");
  static_assert(4 * (3 * BN + 2 * BM) <= S * STAGE, "epilogue staging fits in LDS");
  static_assert(BM * (2 * BN + 8) <= S * STAGE, "bf16 tile fits in the stage buffers");
  constexpr int NP = DEQ ? 3 * BN + 2 * BM : 0;  // epilogue parameters, after the stages
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE + 4 * NP];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t m0, n0;
  f6_tile_origin<BM, BN, GM>(int(blockIdx.x), M, N, &m0, &n0);
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;
  const int KT = K / 128;
  const int64_t lda = f6_row_bytes(K);

  // DMA unit u fills LDS bytes [1 KB u, 1 KB (u + 1)) of the stage, i.e.
  // 16-B chunks 64 u' + l (u' counts within the A or the B tile; tiles are
  // 3 KB per 32 rows, so no unit straddles them): row (64 u' + l) / 6, slot
  // (64 u' + l) % 6, which holds the row's chunk of the same index with the
  // halves swapped on rows with bit 3 set. Waves whose last unit index runs
  // past the end repeat the final unit (same bytes to the same place), so
  // every wave issues LPW loads per stage. The loads are buffer loads
  // against a per-tile descriptor: rows past M (N) and stages past K fall
  // outside the descriptor's range and move no memory.
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  const int64_t rows_a = (M - m0) < BM ? (M - m0) : BM;
  const int64_t rows_b = (N - n0) < BN ? (N - n0) : BN;
  const uint8_t* abase = A + m0 * lda;
  const uint8_t* bbase = B + n0 * lda;
  // Rows are stored in groups of RG: a group holds, stage by stage, the RG
  // rows' 96-byte segments next to each other (RG * 96 contiguous bytes per
  // stage), so one DMA instruction reads whole aligned cache lines.
  const int nrec_a = int((rows_a + RG - 1) / RG * RG * lda);
  const int nrec_b = int((rows_b + RG - 1) / RG * RG * lda);
  uint32_t voff[LPW];
  int ldst[LPW];
#pragma unroll
  for (int q = 0; q < LPW; ++q) {
    int u = q * NW + wv;
    if (u > UNITS - 1) u = UNITS - 1;
    const bool isA = q < QA;
    const int ul = isA ? u : u - UA;
    const int c = 64 * ul + lane;
    const int row = c / 6, slot = c - 6 * (c / 6);
    const int h = (slot >= 3 ? 1 : 0) ^ ((row >> 3) & 1);
    voff[q] = uint32_t((row / RG) * RG * lda + (row % RG) * 96 + 48 * h +
                       16 * (slot - 3 * (slot >= 3 ? 1 : 0)));
    ldst[q] = u * 1024;
  }
#define HQ6_ISSUE(KT_)                                                                    \
  do {                                                                                    \
    const int kt_ = (KT_);                                                                \
    uint8_t* base_ = smem + (kt_ % S) * STAGE;                                            \
    const bool ok_ = kt_ < KT;                                                            \
    const __amdgpu_buffer_rsrc_t ra_ = make_rsrc(abase, ok_ ? nrec_a : 0);                \
    const __amdgpu_buffer_rsrc_t rb_ = make_rsrc(bbase, ok_ ? nrec_b : 0);                \
    _Pragma("unroll") for (int q = 0; q < LPW; ++q)                                       \
        lds_dma16_buf(q < QA ? ra_ : rb_, voff[q], uint32_t(kt_) * (96u * RG), base_ + ldst[q]); \
  } while (0)

  const int lrow = lane & 31, lhalf = lane >> 5;
  const int loff = lrow * 96 + 48 * (lhalf ^ ((lrow >> 3) & 1));
#define HQ6_READ(SET_, KT_)                                                               \
  do {                                                                                    \
    const uint8_t* cur_ = smem + ((KT_) % S) * STAGE + loff;                              \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                        \
      _Pragma("unroll") for (int p = 0; p < 3; ++p) af[SET_][i].c[p] =                    \
          *reinterpret_cast<const v4i*>(cur_ + (wm0 + 32 * i) * 96 + 16 * p);             \
    _Pragma("unroll") for (int j = 0; j < TN; ++j)                                        \
      _Pragma("unroll") for (int p = 0; p < 3; ++p) bf[SET_][j].c[p] =                    \
          *reinterpret_cast<const v4i*>(cur_ + (BM + wn0 + 32 * j) * 96 + 16 * p);        \
  } while (0)
#define HQ6_MFMA(SET_)                                                                    \
  do {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                        \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                    \
        acc[i][j] = mfma_f6(f6_op0(bf[SET_][j]), f6_op0(af[SET_][i]), acc[i][j]);         \
        acc[i][j] = mfma_f6(f6_op1(bf[SET_][j]), f6_op1(af[SET_][i]), acc[i][j]);         \
      }                                                                                   \
  } while (0)
  // One iteration on stage KT_ (fragments in set SET_): wait for stage KT_+1
  // (stage KT_+2 may stay in flight), refill the buffer of stage KT_ with
  // stage KT_+3, prefetch the fragments of stage KT_+1, run the MFMAs. Past
  // the last stage the refills are empty and the prefetched values unused,
  // so every iteration is the same straight sequence.
#define HQ6_FULL(SET_, KT_)                                                               \
  do {                                                                                    \
    wait_vm_lgkm0<LPW>();                                                                 \
    __builtin_amdgcn_s_barrier();                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    HQ6_ISSUE((KT_) + 3);                                                                 \
    HQ6_READ(1 - (SET_), (KT_) + 1);                                                      \
    HQ6_MFMA(SET_);                                                                       \
    mfma_interleave<0, 2 * TM * TN, 3 * (TM + TN), LPW>();                                \
    __builtin_amdgcn_sched_barrier(0);                                                    \
  } while (0)

  v16f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      acc[i][j] = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  Frag6 af[2][TM], bf[2][TN];

  // The epilogue's parameters travel first, so every later wait covers them.
  if constexpr (DEQ) params_dma<BM, BN, NW>(smem + S * STAGE, wv, lane, m0, n0, M, N, ep);
  HQ6_ISSUE(0);
  HQ6_ISSUE(1);
  HQ6_ISSUE(2);
  wait_vm_lgkm0<2 * LPW>();
  __builtin_amdgcn_s_barrier();
  HQ6_READ(0, 0);
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    HQ6_FULL(0, kt);
    HQ6_FULL(1, kt + 1);
  }
  if (kt < KT) HQ6_FULL(0, kt);
  wait_vm_lgkm0<0>();  // no LDS write may land after the block ends
#undef HQ6_FULL
#undef HQ6_MFMA
#undef HQ6_READ
#undef HQ6_ISSUE

  if constexpr (DEQ) {
    if (ep.y_bf16) {
      if (ep.rank)
        gemm_epilogue_bf16_staged<BM, BN, TM, TN, NW, true>(
            acc, smem, reinterpret_cast<const float*>(smem + S * STAGE), tid, lane, m0, n0, wm0,
            wn0, M, N, ep);
      else
        gemm_epilogue_bf16_staged<BM, BN, TM, TN, NW, false>(
            acc, smem, reinterpret_cast<const float*>(smem + S * STAGE), tid, lane, m0, n0, wm0,
            wn0, M, N, ep);
      return;
    }
  }
  gemm_epilogue<BM, BN, TM, TN, NW, DEQ>(acc, smem, tid, lane, m0, n0, wm0, wn0, M, N, Cout, ldc, ep);
}

}  // namespace hq
