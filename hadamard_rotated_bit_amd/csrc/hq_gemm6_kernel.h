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

#include <type_traits>

#include "hq_gemm_kernel.h"

namespace hq {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v2i __attribute__((ext_vector_type(2)));

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

// The same parameters with a fixed unit per wave and array: wave w copies
// unit min(w, units - 1) of each of the five vectors (64 floats per unit;
// repeated units write the same bytes), five loads per wave with no
// wave-dependent control flow.
template <int BM, int BN, int NW>
__device__ __forceinline__ void params_dma_fixed(uint8_t* P, int wv, int lane, int64_t m0,
                                                 int64_t n0, int64_t M, int64_t N,
                                                 const GemmEpi& ep) {
  constexpr int UN = BN / 64, UM = BM / 64;
  static_assert(BN % 64 == 0 && BM % 64 == 0 && UN <= NW && UM <= NW, "one unit per wave");
  const int un = wv < UN ? wv : UN - 1;
  const int um = wv < UM ? wv : UM - 1;
  const int64_t cn = n0 + 64 * un, rm = m0 + 64 * um;
  const int64_t ln = N - cn, lm = M - rm;
  const int bn = int((ln < 64 ? (ln > 0 ? ln : 0) : 64) * 4);
  const int bm = int((lm < 64 ? (lm > 0 ? lm : 0) : 64) * 4);
  const uint32_t vo = uint32_t(lane) * 4u;
  lds_dma4_buf(make_rsrc(ep.s_w + cn, bn), vo, 0u, P + 4 * (64 * un));
  lds_dma4_buf(make_rsrc(ep.c + cn, bn), vo, 0u, P + 4 * (BN + 64 * un));
  lds_dma4_buf(make_rsrc(ep.bias + cn, bn), vo, 0u, P + 4 * (2 * BN + 64 * un));
  lds_dma4_buf(make_rsrc(ep.s_x + rm, bm), vo, 0u, P + 4 * (3 * BN + 64 * um));
  lds_dma4_buf(make_rsrc(ep.mu + rm, bm), vo, 0u, P + 4 * (3 * BN + BM + 64 * um));
}

template <int BM, int BN, int WM, int WN, int S, int GM, bool DEQ, int RG = 1, int OCC = 1>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(OCC))) void gemm_f6_kernel(
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
  static_assert(S == 2 || S == 3, "two or three stage buffers");
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
    wait_vm_lgkm0<(S - 2) * LPW>();                                                       \
    __builtin_amdgcn_s_barrier();                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    HQ6_ISSUE((KT_) + S);                                                                 \
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
  if constexpr (S == 3) HQ6_ISSUE(2);
  wait_vm_lgkm0<(S - 1) * LPW>();
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

// Persistent variant for bf16 outputs (one block of 4 waves per CU, grid at
// most one block per CU): the block walks the tiles blockIdx.x,
// blockIdx.x + gridDim.x, ... with a single stage pipeline across tile
// boundaries. Global stage g (tile g / KT, k-step g % KT) lives in buffer
// g mod S (S = 3 stage buffers for FP6 codes, 4 for int8), so the last S
// iterations of a tile already load the first S stages of the next one and
// those loads overlap the epilogue.
//
// The epilogue does not touch the stage buffers: each wave stages its
// 32-row slices in a private LDS area and writes them back with 16-byte
// buffer stores that always issue (rows past M fall outside the descriptor,
// columns past N get an out-of-range offset); then the next tile's epilogue
// parameters are loaded into the other of two parameter buffers. Every wave
// thus issues, per tile, KT stage loads of LPW instructions, NST stores and
// PPW parameter loads, in a fixed order, and the waits count them (vector
// memory operations retire in issue order): k-steps 0 .. S - 2 may leave the
// previous epilogue's stores and parameter loads in flight
// ((S - 2) LPW + NST + PPW outstanding), later k-steps only the S - 2 stages
// loaded after the one they need ((S - 2) LPW). The prologue issues NST
// stores that move no memory so that the first tile has the same sequence.
// A tile's parameters are retired by its k-step S - 1 (at least S stages per
// tile: K >= 384 for FP6 codes).
//
// The same body serves int8 codes (I8; gemm_i8_persist): a stage is then 64
// codes, i.e. 64-byte rows stored with the int8 kernel's chunk swizzle
// (chunk c of row r in slot c ^ ((r >> 2) & 3): the 16 lanes of a
// ds_read_b128 phase hit 16 distinct 16-byte positions), one 1-KB DMA unit
// holds 16 rows, and each 32-code half of a stage is one
// v_mfma_i32_32x32x32_i8 per 32 x 32 output (int32 accumulators, converted
// to float in the epilogue). Four stage buffers (28 KB each) fit beside the
// staging and parameter areas, so each stage load has three iterations to
// land. K >= 256, K % 64 == 0.
struct Frag8 {
  v4i c[2];
};
template <bool I8, int BM, int BN, int WM, int WN, int GM, int RG, int LR>
__device__ __forceinline__ void persist_body(const uint8_t* __restrict__ A, int64_t M,
                                             const uint8_t* __restrict__ B, int64_t N, int K,
                                             GemmEpi ep) {
  // stage buffers: three 43-KB FP6 stages, four 28-KB int8 stages
  constexpr int S = I8 ? 4 : 3;
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int WAVES_N = BN / WN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int RB = I8 ? 64 : 96;             // bytes of a row per stage
  constexpr int KS = I8 ? 64 : 128;            // codes per stage
  constexpr int STAGE = RB * (BM + BN);
  constexpr int UA = I8 ? BM / 16 : 3 * BM / 32;
  constexpr int UNITS = I8 ? (BM + BN) / 16 : 3 * (BM + BN) / 32;
  constexpr int LPW = (UNITS + NW - 1) / NW;
  constexpr int QA = UA / NW;
  constexpr int NP = 3 * BN + 2 * BM;          // floats per parameter buffer
  constexpr int PPW = 5;                       // loads per params_dma_fixed
  constexpr int CPR = WN / 8;                  // 16-byte pieces per slice row
  constexpr int SP = 2 * WN + 8;               // staging pitch (bytes)
  constexpr int SPS = 32 * CPR / 64;           // stores per slice
  constexpr int NST = TM * SPS;                // stores per wave and tile
  // outstanding vector-memory operations a k-step's wait allows: the S - 2
  // stages loaded after the one it needs, plus, in the first S - 1 k-steps
  // of a tile, the previous epilogue's stores and parameter loads
  constexpr int WSTEP = (S - 2) * LPW;
  constexpr int WBIG = WSTEP + NST + PPW;
  static_assert(UA % NW == 0 && BM % 32 == 0 && BN % 32 == 0, "whole 1-KB units per tile");
  static_assert((32 * CPR) % 64 == 0, "whole store instructions per slice");
  static_assert((S - 1) * LPW + NST + PPW <= 63, "outstanding count fits vmcnt");
  static_assert((((SP / 4) % 64) & 3) == 2, "staging pitch = 2 x odd dwords mod 64 banks");
  // LDS: two parameter buffers, the waves' staging areas, the stage buffers
  // (the epilogue's accesses keep small constant offsets).
  constexpr int SB = 2 * 4 * NP + NW * 32 * SP;
  static_assert(SB % 256 == 0, "stage buffers start on a bank line");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[SB + S * STAGE];
  uint8_t* const smem = lds + SB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wv = __builtin_amdgcn_readfirstlane(wave);
  uint8_t* const stg = lds + 2 * 4 * NP + wv * 32 * SP;
  const int wm0 = (wv / WAVES_N) * WM, wn0 = (wv % WAVES_N) * WN;
  const int KT = K / KS;
  const int64_t lda = I8 ? int64_t(K) : f6_row_bytes(K);
  const int ntiles = int((M + BM - 1) / BM) * int((N + BN - 1) / BN);
  const int G = int(gridDim.x);

  // Three 1-KB units cover 32 rows exactly (192 chunks of 16 B), so the
  // global offset of unit 3t + r is that of unit r plus 32 t rows: each
  // lane keeps the offsets of units 0, 1 and 2 only.
  // (int8: every unit holds 16 whole rows and lane l always fetches row
  // l / 4 of it, global chunk (l % 4) ^ ((l / 16) % 4): one offset, vb[0].)
  static_assert(I8 || (UA % 3 == 0 && 32 % RG == 0), "unit triples are whole row groups");
  static_assert(UA % NW == 0, "A units split evenly over the waves");
  uint32_t vb[3];
  if constexpr (I8) {
    vb[0] = uint32_t((lane >> 2) * lda + 16 * ((lane & 3) ^ ((lane >> 4) & 3)));
    vb[1] = vb[2] = vb[0];
  } else {
#pragma unroll
    for (int r = 0; r < 3; ++r) {
      const int c = 64 * r + lane;
      const int row = c / 6, slot = c - 6 * (c / 6);
      const int h = (slot >= 3 ? 1 : 0) ^ ((row >> 3) & 1);
      vb[r] = uint32_t((row / RG) * RG * lda + (row % RG) * 96 + 48 * h +
                       16 * (slot - 3 * (slot >= 3 ? 1 : 0)));
    }
  }

  // Source rows of a tile: base pointers and descriptor sizes (0 past the end).
  struct Src {
    const uint8_t* a;
    const uint8_t* b;
    int na, nb;
    int64_t m0, n0;
  };
  auto tile_src = [&](int t) {
    Src r{A, B, 0, 0, 0, 0};
    if (t < ntiles) {
      f6_tile_origin<BM, BN, GM>(t, M, N, &r.m0, &r.n0);
      const int64_t ra = (M - r.m0) < BM ? (M - r.m0) : BM;
      const int64_t rb = (N - r.n0) < BN ? (N - r.n0) : BN;
      r.a = A + r.m0 * lda;
      r.b = B + r.n0 * lda;
      r.na = int((ra + RG - 1) / RG * RG * lda);
      r.nb = int((rb + RG - 1) / RG * RG * lda);
    }
    return r;
  };

  int tile = int(blockIdx.x);
  Src cur = tile_src(tile), nxt = tile_src(tile + G);
  int bufc = 0;  // buffer of the current global stage
  int pb = 0;    // parameter buffer of the current tile

  // Load of k-step KS_ of the current tile (past its end: of the next tile).
#define HP_ISSUE(KS_, BUF_)                                                               \
  do {                                                                                    \
    const int k3_ = (KS_);                                                                \
    const bool nx_ = k3_ >= KT;                                                           \
    const int ks_ = nx_ ? k3_ - KT : k3_;                                                 \
    const __amdgpu_buffer_rsrc_t ra_ = make_rsrc(nx_ ? nxt.a : cur.a, nx_ ? nxt.na : cur.na); \
    const __amdgpu_buffer_rsrc_t rb_ = make_rsrc(nx_ ? nxt.b : cur.b, nx_ ? nxt.nb : cur.nb); \
    uint8_t* base_ = smem + (BUF_) * STAGE;                                               \
    _Pragma("unroll") for (int q = 0; q < LPW; ++q) {                                     \
      int u_ = q * NW + wv;                                                               \
      if (u_ > UNITS - 1) u_ = UNITS - 1;                                                 \
      const int ul_ = q < QA ? u_ : u_ - UA;                                              \
      if constexpr (I8) {                                                                 \
        lds_dma16_buf(q < QA ? ra_ : rb_, vb[0],                                          \
                      uint32_t(ks_) * 64u + uint32_t(ul_) * uint32_t(16 * lda),           \
                      base_ + u_ * 1024);                                                 \
      } else {                                                                            \
        const int t_ = ul_ / 3, r_ = ul_ - 3 * t_;                                        \
        const uint32_t vo_ = (r_ == 0 ? vb[0] : (r_ == 1 ? vb[1] : vb[2])) +              \
                             uint32_t(t_) * uint32_t(32 * lda);                           \
        lds_dma16_buf(q < QA ? ra_ : rb_, vo_, uint32_t(ks_) * (96u * RG),                \
                      base_ + u_ * 1024);                                                 \
      }                                                                                   \
    }                                                                                     \
  } while (0)

  const int lrow = lane & 31, lhalf = lane >> 5;
  // FP6: the lane's 48 bytes of its row (halves swapped on rows with bit 3);
  // int8: chunk p (0, 1) of the lane's 32-code half h is global chunk
  // 2 p + h, stored in slot (2 p + h) ^ ((row >> 2) & 3) (every 32-row block
  // starts on a multiple of 4 rows, so the slot depends on lrow only).
  const int loff = I8 ? lrow * 64 : lrow * 96 + 48 * (lhalf ^ ((lrow >> 3) & 1));
  const int lsl0 = 16 * ((0 + lhalf) ^ ((lrow >> 2) & 3));
  const int lsl1 = 16 * ((2 + lhalf) ^ ((lrow >> 2) & 3));
#define HP_READ(SET_, BUF_)                                                               \
  do {                                                                                    \
    const uint8_t* cur_ = smem + (BUF_) * STAGE + loff;                                   \
    if constexpr (I8) {                                                                   \
      _Pragma("unroll") for (int i = 0; i < TM; ++i) {                                    \
        af[SET_][i].c[0] = *reinterpret_cast<const v4i*>(cur_ + (wm0 + 32 * i) * 64 + lsl0); \
        af[SET_][i].c[1] = *reinterpret_cast<const v4i*>(cur_ + (wm0 + 32 * i) * 64 + lsl1); \
      }                                                                                   \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                    \
        bf[SET_][j].c[0] = *reinterpret_cast<const v4i*>(cur_ + (BM + wn0 + 32 * j) * 64 + lsl0); \
        bf[SET_][j].c[1] = *reinterpret_cast<const v4i*>(cur_ + (BM + wn0 + 32 * j) * 64 + lsl1); \
      }                                                                                   \
    } else {                                                                              \
      _Pragma("unroll") for (int i = 0; i < TM; ++i)                                      \
        _Pragma("unroll") for (int p = 0; p < 3; ++p) af[SET_][i].c[p] =                  \
            *reinterpret_cast<const v4i*>(cur_ + (wm0 + 32 * i) * 96 + 16 * p);           \
      _Pragma("unroll") for (int j = 0; j < TN; ++j)                                      \
        _Pragma("unroll") for (int p = 0; p < 3; ++p) bf[SET_][j].c[p] =                  \
            *reinterpret_cast<const v4i*>(cur_ + (BM + wn0 + 32 * j) * 96 + 16 * p);      \
    }                                                                                     \
  } while (0)
#define HP_MFMA(SET_)                                                                     \
  do {                                                                                    \
    _Pragma("unroll") for (int i = 0; i < TM; ++i)                                        \
      _Pragma("unroll") for (int j = 0; j < TN; ++j) {                                    \
        if constexpr (I8) {                                                               \
          _Pragma("unroll") for (int p = 0; p < 2; ++p) acc[i][j] =                       \
              __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[SET_][j].c[p], af[SET_][i].c[p],   \
                                                    acc[i][j], 0, 0, 0);                  \
        } else {                                                                          \
          acc[i][j] = mfma_f6(f6_op0(bf[SET_][j]), f6_op0(af[SET_][i]), acc[i][j]);       \
          acc[i][j] = mfma_f6(f6_op1(bf[SET_][j]), f6_op1(af[SET_][i]), acc[i][j]);       \
        }                                                                                 \
      }                                                                                   \
  } while (0)
  // One iteration on k-step KT_ of the current tile (fragments in SET_):
  // wait for the next global stage, join the block, refill the current
  // buffer with the stage S ahead, prefetch the fragments of the next
  // global stage (at the tile's last k-step: the next tile's first), run the
  // MFMAs.
#define HP_STEP(SET_, KT_)                                                                \
  do {                                                                                    \
    if ((KT_) < S - 1) wait_vm_lgkm0<WBIG>(); else wait_vm_lgkm0<WSTEP>();                \
    __builtin_amdgcn_s_barrier();                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    const int bn_ = bufc == S - 1 ? 0 : bufc + 1;                                         \
    HP_ISSUE((KT_) + S, bufc);                                                            \
    HP_READ(1 - (SET_), bn_);                                                             \
    HP_MFMA(SET_);                                                                        \
    mfma_interleave<0, 2 * TM * TN, (I8 ? 2 : 3) * (TM + TN), LPW>();                     \
    __builtin_amdgcn_sched_barrier(0);                                                    \
    bufc = bn_;                                                                           \
  } while (0)

  using Acc = std::conditional_t<I8, v16i, v16f>;
  using Frag = std::conditional_t<I8, Frag8, Frag6>;
  Acc acc[TM][TN];
  Frag af[2][TM], bf[2][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
      acc[i][j] = Acc{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};

  HP_ISSUE(0, 0);
  HP_ISSUE(1, 1);
  HP_ISSUE(2, 2);
  if constexpr (S == 4) HP_ISSUE(3, 3);
  {
    const __amdgpu_buffer_rsrc_t none = make_rsrc(ep.Y, 0);
    const v4i z = v4i{0, 0, 0, 0};
#pragma unroll
    for (int q = 0; q < NST; ++q) __builtin_amdgcn_raw_buffer_store_b128(z, none, 16 * q, 0, 0);
  }
  params_dma_fixed<BM, BN, NW>(lds, wv, lane, cur.m0, cur.n0, M, N, ep);
  wait_vm_lgkm0<(S - 1) * LPW + NST + PPW>();
  __builtin_amdgcn_s_barrier();
  HP_READ(0, 0);
  for (;;) {
    int kt = 0;
    for (; kt + 1 < KT; kt += 2) {
      HP_STEP(0, kt);
      HP_STEP(1, kt + 1);
    }
    if (kt < KT) {
      HP_STEP(0, kt);
      // odd KT: the next tile's first fragments went to set 1
#pragma unroll
      for (int i = 0; i < TM; ++i) af[0][i] = af[1][i];
#pragma unroll
      for (int j = 0; j < TN; ++j) bf[0][j] = bf[1][j];
    }

    // Epilogue: Y = acc s_x s_w + mu c + b (+ U L2), per 32-row slice of the
    // wave's sub-tile, staged in the wave's LDS area.
    {
      // The lane index is passed through an empty asm statement so that the
      // lane-dependent addresses below are formed per tile instead of being
      // hoisted out of the tile loop (and held in registers across it).
      int el = lane;
      asm volatile("" : "+v"(el));
      const int erow = el & 31, ehalf = el >> 5;
      const float* const Pf = reinterpret_cast<const float*>(lds + pb * 4 * NP);
      const int64_t mw = cur.m0 + wm0;
      const int64_t rem = M - mw;
      const int rows_v = rem <= 0 ? 0 : (rem < WM ? int(rem) : WM);
      const int64_t cl = N - (cur.n0 + wn0);
      const int ncols = cl <= 0 ? 0 : (cl < WN ? int(cl) : WN);  // valid columns of the wave
      uint16_t* const ybase = static_cast<uint16_t*>(ep.Y) + mw * ep.ldy + (cur.n0 + wn0);
      const __amdgpu_buffer_rsrc_t yr = make_rsrc(ybase, int(rows_v * ep.ldy * 2));
      const int ypitch = int(ep.ldy * 2);
      // Rank <= 32 (one 32-rank chunk): the wave's L2 operands are the same
      // for every slice, so they are loaded once per tile, and U of slice
      // i + 1 is loaded while slice i is computed. LR == 1: L2 was given in
      // bf16, so its low half is zero and takes neither registers nor
      // products; LR == 2: L2 is carried as bf16 hi + lo.
      const bool lr_one = LR != 0 && ep.rank <= 32;
      const bool lr_two = LR != 0 && ep.rank > 16;
      v8bf wh1[LR ? TN : 1][2], wl1[LR == 2 ? TN : 1][2];
      float un[2][8];
      auto load_u = [&](int i_, float (&dst)[2][8]) {
        const int64_t m = mw + i_ * 32 + erow;
        const int64_t mc = m < M ? m : M - 1;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k0 = (h == 0 || lr_two) ? 16 * h : 0;
          load8(ep.U + mc * ep.rank + k0 + 8 * ehalf, dst[h]);
        }
      };
      if constexpr (LR != 0) {
        if (lr_one) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const int k0 = (h == 0 || lr_two) ? 16 * h : 0;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
              const int64_t nb = cur.n0 + wn0 + j * 32;
              const int64_t nr = nb + erow < N ? nb + erow : N - 1;
              const int64_t off = nr * ep.rank + k0 + 8 * ehalf;
              wh1[j][h] = *reinterpret_cast<const v8bf*>(ep.l2_hi + off);
              if constexpr (LR == 2) wl1[j][h] = *reinterpret_cast<const v8bf*>(ep.l2_lo + off);
            }
          }
          load_u(0, un);
        }
      }
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const float sx = Pf[3 * BN + wm0 + 32 * i + erow];
        const float mu = Pf[3 * BN + BM + wm0 + 32 * i + erow];
        // Low-rank term of slice i (all strips): one 32-rank chunk of U and
        // L2 operands loaded before any product (see the tiled epilogue).
        v16f lr[LR ? TN : 1];
        if constexpr (LR != 0) {
          const int64_t m = mw + i * 32 + erow;
          const int64_t mc = m < M ? m : M - 1;
#pragma unroll
          for (int j = 0; j < TN; ++j) lr[j] = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
          if (lr_one) {
            float uf[2][8];
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
              for (int e = 0; e < 8; ++e) uf[h][e] = un[h][e];
            if (i + 1 < TM) load_u(i + 1, un);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              if (h == 1 && !lr_two) break;
              const v8bf uh = pack_bf16x8(uf[h], false), ul = pack_bf16x8(uf[h], true);
#pragma unroll
              for (int j = 0; j < TN; ++j) {
                lr[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh1[j][h], uh, lr[j], 0, 0, 0);
                if constexpr (LR == 2)
                  lr[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl1[j][h], uh, lr[j], 0, 0, 0);
                lr[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh1[j][h], ul, lr[j], 0, 0, 0);
              }
            }
          }
          for (int kc = 0; !lr_one && kc < ep.rank; kc += 32) {
            const bool two = kc + 16 < ep.rank;
            float uf[2][8];
            v8bf wh[TN][2], wl[LR == 2 ? TN : 1][2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const int k0 = (h == 0 || two) ? kc + 16 * h : kc;
              load8(ep.U + mc * ep.rank + k0 + 8 * ehalf, uf[h]);
#pragma unroll
              for (int j = 0; j < TN; ++j) {
                const int64_t nb = cur.n0 + wn0 + j * 32;
                const int64_t nr = nb + erow < N ? nb + erow : N - 1;
                const int64_t off = nr * ep.rank + k0 + 8 * ehalf;
                wh[j][h] = *reinterpret_cast<const v8bf*>(ep.l2_hi + off);
                if constexpr (LR == 2) wl[j][h] = *reinterpret_cast<const v8bf*>(ep.l2_lo + off);
              }
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              if (h == 1 && !two) break;
              const v8bf uh = pack_bf16x8(uf[h], false), ul = pack_bf16x8(uf[h], true);
#pragma unroll
              for (int j = 0; j < TN; ++j) {
                lr[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh[j][h], uh, lr[j], 0, 0, 0);
                if constexpr (LR == 2)
                  lr[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl[j][h], uh, lr[j], 0, 0, 0);
                lr[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh[j][h], ul, lr[j], 0, 0, 0);
              }
            }
          }
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          // Parameters are re-read from LDS per slice and column group (a
          // compiler barrier keeps them from being held across the slices).
          asm volatile("" ::: "memory");
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int nl = wn0 + j * 32 + 8 * g + 4 * ehalf;
            const float4 sw = make_float4(Pf[nl], Pf[nl+1], Pf[nl+2], Pf[nl+3]);
            const float4 cb = make_float4(Pf[BN+nl], Pf[BN+nl+1], Pf[BN+nl+2], Pf[BN+nl+3]);
            const float4 bb = make_float4(Pf[2*BN+nl], Pf[2*BN+nl+1], Pf[2*BN+nl+2], Pf[2*BN+nl+3]);
            const Acc& a = acc[i][j];
            float y0 = fmaf(float(a[4 * g + 0]), sx * sw.x, fmaf(mu, cb.x, bb.x));
            float y1 = fmaf(float(a[4 * g + 1]), sx * sw.y, fmaf(mu, cb.y, bb.y));
            float y2 = fmaf(float(a[4 * g + 2]), sx * sw.z, fmaf(mu, cb.z, bb.z));
            float y3 = fmaf(float(a[4 * g + 3]), sx * sw.w, fmaf(mu, cb.w, bb.w));
            if constexpr (LR != 0) {
              y0 += lr[j][4 * g + 0];
              y1 += lr[j][4 * g + 1];
              y2 += lr[j][4 * g + 2];
              y3 += lr[j][4 * g + 3];
            }
            {
              const uint32_t la = uint32_t(reinterpret_cast<uintptr_t>(stg + erow * SP + (j * 32 + 8 * g + 4 * ehalf) * 2));
              const uint2 dv = make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
              asm volatile("ds_write_b64 %0, %1" :: "v"(la), "v"(dv) : "memory");
            }
          }
        }
        static_assert(SPS == 6, "six pieces per lane and slice");
        uint32_t la[SPS];
        uint32_t off[SPS];
#pragma unroll
        for (int s = 0; s < SPS; ++s) {
          const int q = el + 64 * s, r = q / CPR, ch = q - r * CPR;
          la[s] = uint32_t(reinterpret_cast<uintptr_t>(stg + r * SP + ch * 16));
          const bool ok = ch * 8 < ncols;
          off[s] = ok ? uint32_t((32 * i + r) * ypitch + ch * 16) : 0x80000000u;
        }
        v4i d0, d1, d2, d3, d4, d5;
        asm volatile(
            "ds_read2_b64 %0, %6 offset1:1\n"
            "ds_read2_b64 %1, %7 offset1:1\n"
            "ds_read2_b64 %2, %8 offset1:1\n"
            "ds_read2_b64 %3, %9 offset1:1\n"
            "ds_read2_b64 %4, %10 offset1:1\n"
            "ds_read2_b64 %5, %11 offset1:1\n"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(d0), "=&v"(d1), "=&v"(d2), "=&v"(d3), "=&v"(d4), "=&v"(d5)
            : "v"(la[0]), "v"(la[1]), "v"(la[2]), "v"(la[3]), "v"(la[4]), "v"(la[5])
            : "memory");
        __builtin_amdgcn_raw_buffer_store_b128(d0, yr, off[0], 0, Y_STORE_CPOL);
        __builtin_amdgcn_raw_buffer_store_b128(d1, yr, off[1], 0, Y_STORE_CPOL);
        __builtin_amdgcn_raw_buffer_store_b128(d2, yr, off[2], 0, Y_STORE_CPOL);
        __builtin_amdgcn_raw_buffer_store_b128(d3, yr, off[3], 0, Y_STORE_CPOL);
        __builtin_amdgcn_raw_buffer_store_b128(d4, yr, off[4], 0, Y_STORE_CPOL);
        __builtin_amdgcn_raw_buffer_store_b128(d5, yr, off[5], 0, Y_STORE_CPOL);
      }
    }
    // The next tile's parameters go to the other buffer (nobody reads it:
    // its last reader was the epilogue two tiles back).
    pb ^= 1;
    params_dma_fixed<BM, BN, NW>(lds + pb * 4 * NP, wv, lane, nxt.m0, nxt.n0, M, N, ep);

    tile += G;
    if (tile >= ntiles) break;
    cur = nxt;
    nxt = tile_src(tile + G);
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j)
        acc[i][j] = Acc{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  }
  wait_vm_lgkm0<0>();  // no LDS write may land after the block ends
#undef HP_STEP
#undef HP_MFMA
#undef HP_READ
#undef HP_ISSUE
}

template <int BM, int BN, int WM, int WN, int GM, int RG, int LR>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(1))) void gemm_f6_persist(
    const uint8_t* __restrict__ A, int64_t M, const uint8_t* __restrict__ B, int64_t N, int K,
    GemmEpi ep) {
  persist_body<false, BM, BN, WM, WN, GM, RG, LR>(A, M, B, N, K, ep);
}

template <int BM, int BN, int WM, int WN, int GM, int LR>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(1))) void gemm_i8_persist(
    const uint8_t* __restrict__ A, int64_t M, const uint8_t* __restrict__ B, int64_t N, int K,
    GemmEpi ep) {
  persist_body<true, BM, BN, WM, WN, GM, 1, LR>(A, M, B, N, K, ep);
}

}  // namespace hq
