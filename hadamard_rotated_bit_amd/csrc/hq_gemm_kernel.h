// Int8 MFMA GEMM kernel template of libhq (gfx950), shared by the library and
// its tuning harness. See hq_gemm.hip for the operation and the epilogue.
#pragma once

#include "hq_device.h"
#include "hq_gemm_types.h"

namespace hq {

// LDS holds each stage tile as rows of BK bytes (NC = BK/16 chunks of 16 B).
// gfx950 LDS serves 16 lanes x 16 B per clock from 64 four-byte banks, so the
// 16 lanes that read one chunk column of 16 consecutive rows must land in 16
// distinct 16-B positions of a 256-B bank line. Chunk c of row r is therefore
// stored at slot c ^ ((r >> SH) mod NC) with SH = log2(256 / BK): rows that
// share a bank line differ in their row offset, and the next SH bits of the
// row index permute the chunk slot.
template <int BK>
__device__ __forceinline__ int swz(int row, int chunk) {
  constexpr int NC = BK / 16;
  constexpr int SH = (BK == 128) ? 1 : 2;
  return row * BK + ((chunk ^ ((row >> SH) & (NC - 1))) << 4);
}

// Raw buffer descriptor over `bytes` bytes at `base` (stride 0; gfx9 data
// format word): loads at offsets >= bytes return without touching memory, stores there are
// dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, bytes, 0x00020000);
}

// Cache policy of the output stores (sc0 sc1: system scope). Y is written
// once and never read back by the kernel, so its lines are written through
// to memory instead of being kept in L2, where they would evict the operand
// lines the other tiles of the XCD still read.
constexpr int Y_STORE_CPOL = 17;

// s_waitcnt with vmcnt = N (vector-memory ops still allowed in flight) and
// lgkmcnt = 0 (every LDS read issued by this wave has returned).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// 8 floats -> 8 bf16 (round to nearest even); `residual` gives the bf16 of
// what the first rounding left over, so hi + lo carries ~16 significant bits.
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

// Epilogue shared by the GEMM kernels (int32 or exact-integer float
// accumulators): lane owns token
// m = m0 + wm0 + 32 i + l % 32 and, per 32-column strip j, channels
// n = n0 + wn0 + 32 j + 8 g + 4 (l / 32) + {0..3}, g = 0..3. `smem` must be
// idle (no LDS reads or DMA of the main loop in flight in any wave) once
// every wave of the block has arrived; its first 4 (3 BN + 2 BM) bytes are
// reused for the block's per-channel and per-token vectors.
template <int BM, int BN, int TM, int TN, int NW, bool DEQ, typename AccT>
__device__ __forceinline__ void gemm_epilogue(AccT (&acc)[TM][TN], uint8_t* smem, int tid, int lane,
                                              int64_t m0, int64_t n0, int wm0, int wn0, int64_t M,
                                              int64_t N, int32_t* __restrict__ Cout, int64_t ldc,
                                              const GemmEpi& ep) {
  const int lrow = lane & 31, lhalf = lane >> 5;
  if constexpr (!DEQ) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + wm0 + i * 32 + lrow;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int64_t n = n0 + wn0 + j * 32 + 8 * g + 4 * lhalf;
          if (m < M && n < N) {
            const AccT& a = acc[i][j];
            *reinterpret_cast<int4*>(Cout + m * ldc + n) =
                make_int4(int(a[4 * g]), int(a[4 * g + 1]), int(a[4 * g + 2]), int(a[4 * g + 3]));
          }
        }
    }
  } else {
    // The block's per-channel vectors (s_w, c, b for BN channels) and
    // per-token vectors (s_x, mu for BM tokens) are staged once in the now
    // idle LDS; lanes then read them as broadcast LDS loads (32 lanes share
    // each channel quadruple) instead of re-fetching them from memory.
    float* P = reinterpret_cast<float*>(smem);
    wait_vm_lgkm0<0>();
    __builtin_amdgcn_s_barrier();
    // (prescaled accumulators: unit scales, so y = acc + b + mu c exactly)
    for (int idx = tid; idx < BN; idx += NW * 64) {
      const int64_t nc = n0 + idx < N ? n0 + idx : N - 1;
      P[idx] = ep.prescaled ? 1.0f : ep.s_w[nc];
      P[BN + idx] = ep.c[nc];
      P[2 * BN + idx] = ep.bias[nc];
    }
    for (int idx = tid; idx < BM; idx += NW * 64) {
      const int64_t mc = m0 + idx < M ? m0 + idx : M - 1;
      P[3 * BN + idx] = ep.prescaled ? 1.0f : ep.s_x[mc];
      P[3 * BN + BM + idx] = ep.mu[mc];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int ml = wm0 + i * 32 + lrow;
      const int64_t m = m0 + ml;
      const int64_t mc = m < M ? m : M - 1;
      const float sx = P[3 * BN + ml], mu = P[3 * BN + BM + ml];
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int64_t nb = n0 + wn0 + j * 32;
        // Low-rank term U[m, :] . L2[:, n] on bf16 MFMA with split operands:
        // first operand L2^T (rows = channels), second U (columns = tokens),
        // so the fp32 result has the accumulator's layout.
        v16f lr = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
        for (int k0 = 0; k0 < ep.rank; k0 += 16) {
          float f[8];
          load8(ep.U + mc * ep.rank + k0 + 8 * lhalf, f);
          const v8bf uh = pack_bf16x8(f, false), ul = pack_bf16x8(f, true);
          const int64_t nr = nb + lrow < N ? nb + lrow : N - 1;
          const int64_t off = nr * ep.rank + k0 + 8 * lhalf;
          const v8bf wh = *reinterpret_cast<const v8bf*>(ep.l2_hi + off);
          lr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh, uh, lr, 0, 0, 0);
          if (!ep.l2_lo_zero) {
            const v8bf wl = *reinterpret_cast<const v8bf*>(ep.l2_lo + off);
            lr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl, uh, lr, 0, 0, 0);
          }
          lr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh, ul, lr, 0, 0, 0);
        }
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int nl = wn0 + j * 32 + 8 * g + 4 * lhalf;
          const int64_t n = n0 + nl;
          const float4 sw = *reinterpret_cast<const float4*>(P + nl);
          const float4 cb = *reinterpret_cast<const float4*>(P + BN + nl);
          const float4 bb = *reinterpret_cast<const float4*>(P + 2 * BN + nl);
          const AccT& a = acc[i][j];
          const float y0 = fmaf(float(a[4 * g + 0]), sx * sw.x, fmaf(mu, cb.x, bb.x)) + lr[4 * g + 0];
          const float y1 = fmaf(float(a[4 * g + 1]), sx * sw.y, fmaf(mu, cb.y, bb.y)) + lr[4 * g + 1];
          const float y2 = fmaf(float(a[4 * g + 2]), sx * sw.z, fmaf(mu, cb.z, bb.z)) + lr[4 * g + 2];
          const float y3 = fmaf(float(a[4 * g + 3]), sx * sw.w, fmaf(mu, cb.w, bb.w)) + lr[4 * g + 3];
          if (m < M && n < N) {
            if (ep.y_bf16) {
              const uint32_t p0 = uint32_t(f32_to_bf16(y0)) | (uint32_t(f32_to_bf16(y1)) << 16);
              const uint32_t p1 = uint32_t(f32_to_bf16(y2)) | (uint32_t(f32_to_bf16(y3)) << 16);
              *reinterpret_cast<uint2*>(static_cast<uint16_t*>(ep.Y) + m * ep.ldy + n) =
                  make_uint2(p0, p1);
            } else {
              *reinterpret_cast<float4*>(static_cast<float*>(ep.Y) + m * ep.ldy + n) =
                  make_float4(y0, y1, y2, y3);
            }
          }
        }
      }
    }
  }
}

// Dequant epilogue with bf16 output staged through LDS (same values as
// gemm_epilogue), with the block's parameters already in LDS at P (laid out
// as in gemm_epilogue, outside the first BM (2 BN + 8) bytes): each lane writes its 4-channel runs (8 bytes) into a
// block-sized bf16 tile in LDS with a row pitch of 2 BN + 8 bytes (the 32
// rows written by one ds_write_b64 phase then fall on 32 distinct bank
// pairs), and the block copies the tile out row by row in 16-byte pieces, so
// every global store instruction writes whole contiguous row segments.
// Loops run channel quadruple outermost, so the per-channel parameters are
// read from LDS once per quadruple and reused for the lane's TM tokens; LR
// selects the low-rank term at compile time. The main loop's LDS must be
// idle.
template <int BM, int BN, int TM, int TN, int NW, bool LR, typename AccT>
__device__ __forceinline__ void gemm_epilogue_bf16_staged(AccT (&acc)[TM][TN], uint8_t* smem,
                                                          const float* P, int tid, int lane,
                                                          int64_t m0, int64_t n0, int wm0, int wn0,
                                                          int64_t M, int64_t N, const GemmEpi& ep) {
  constexpr int PITCH = 2 * BN + 8;
  static_assert((((PITCH / 4) % 64) & 3) == 2, "pitch = 2 x odd dwords mod 64 banks");
  uint8_t* tile = smem;
  const int lrow = lane & 31, lhalf = lane >> 5;
  wait_vm_lgkm0<0>();
  __builtin_amdgcn_s_barrier();
  float sx[TM], mu[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    sx[i] = P[3 * BN + wm0 + i * 32 + lrow];
    mu[i] = P[3 * BN + BM + wm0 + i * 32 + lrow];
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    v16f lr[LR ? TM : 1];
    if constexpr (LR) {
      // Low-rank term of strip j for the wave's TM row slices, 32 ranks at a
      // time: every U and L2 operand of a 32-rank chunk is loaded before the
      // first is used (one memory round trip per chunk; the U loads do not
      // depend on j). A missing second half (rank 16) reloads the first and
      // skips its products.
      const int64_t nb = n0 + wn0 + j * 32;
      const int64_t nr = nb + lrow < N ? nb + lrow : N - 1;
#pragma unroll
      for (int i = 0; i < TM; ++i) lr[i] = v16f{0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
      for (int kc = 0; kc < ep.rank; kc += 32) {
        const bool two = kc + 16 < ep.rank;
        float uf[TM][2][8];
        v8bf wh[2], wl[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int k0 = (h == 0 || two) ? kc + 16 * h : kc;
          const int64_t off = nr * ep.rank + k0 + 8 * lhalf;
          wh[h] = *reinterpret_cast<const v8bf*>(ep.l2_hi + off);
          wl[h] = ep.l2_lo_zero ? wh[h] : *reinterpret_cast<const v8bf*>(ep.l2_lo + off);
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int64_t m = m0 + wm0 + i * 32 + lrow;
            const int64_t mc = m < M ? m : M - 1;
            load8(ep.U + mc * ep.rank + k0 + 8 * lhalf, uf[i][h]);
          }
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (h == 1 && !two) break;
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const v8bf uh = pack_bf16x8(uf[i][h], false), ul = pack_bf16x8(uf[i][h], true);
            lr[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh[h], uh, lr[i], 0, 0, 0);
            if (!ep.l2_lo_zero)
              lr[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wl[h], uh, lr[i], 0, 0, 0);
            lr[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wh[h], ul, lr[i], 0, 0, 0);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int nl = wn0 + j * 32 + 8 * g + 4 * lhalf;
      const float4 sw = *reinterpret_cast<const float4*>(P + nl);
      const float4 cb = *reinterpret_cast<const float4*>(P + BN + nl);
      const float4 bb = *reinterpret_cast<const float4*>(P + 2 * BN + nl);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const AccT& a = acc[i][j];
        float y0 = fmaf(float(a[4 * g + 0]), sx[i] * sw.x, fmaf(mu[i], cb.x, bb.x));
        float y1 = fmaf(float(a[4 * g + 1]), sx[i] * sw.y, fmaf(mu[i], cb.y, bb.y));
        float y2 = fmaf(float(a[4 * g + 2]), sx[i] * sw.z, fmaf(mu[i], cb.z, bb.z));
        float y3 = fmaf(float(a[4 * g + 3]), sx[i] * sw.w, fmaf(mu[i], cb.w, bb.w));
        if constexpr (LR) {
          y0 += lr[i][4 * g + 0];
          y1 += lr[i][4 * g + 1];
          y2 += lr[i][4 * g + 2];
          y3 += lr[i][4 * g + 3];
        }
        const int ml = wm0 + i * 32 + lrow;
        *reinterpret_cast<uint2*>(tile + ml * PITCH + nl * 2) =
            make_uint2(pack_bf16x2(y0, y1), pack_bf16x2(y2, y3));
      }
    }
  }
  __syncthreads();
  constexpr int CPR = BN / 8;  // 16-byte pieces per tile row
  // the tile's rows of Y (m0 < M for every launched tile)
  const int64_t rows_v = M - m0 < BM ? M - m0 : BM;
  const __amdgpu_buffer_rsrc_t yr =
      make_rsrc(static_cast<uint16_t*>(ep.Y) + m0 * ep.ldy, int(rows_v * ep.ldy * 2));
#pragma unroll 8
  for (int q = tid; q < BM * CPR; q += NW * 64) {
    const int row = q / CPR, ch = q - row * CPR;
    const int64_t m = m0 + row, n = n0 + ch * 8;
    if (m < M && n < N) {
      const uint8_t* src = tile + row * PITCH + ch * 16;
      const uint2 lo = *reinterpret_cast<const uint2*>(src);
      const uint2 hi = *reinterpret_cast<const uint2*>(src + 8);
      __builtin_amdgcn_raw_buffer_store_b128(v4i{int(lo.x), int(lo.y), int(hi.x), int(hi.y)}, yr,
                                             uint32_t((row * ep.ldy + n) * 2), 0, Y_STORE_CPOL);
    }
  }
}

// Main loop
// ---------
// Stage loads go straight from global memory to LDS (gfx950
// global_load_lds_dwordx4): one instruction moves 64 lanes x 16 B into 1 KB of
// consecutive LDS, lane l landing in slot l, so the lane fetches the global
// chunk that belongs in that swizzled slot. Waits and barriers are explicit
// (bare s_barrier): stage kt+S-1 is issued right after the barrier that
// retires stage kt-1, so S-1 stages are in flight behind the MFMAs. Inside a
// stage the MFMA fragments of k-step s+1 are read from LDS while the MFMAs of
// step s run (two register sets).
//
// The MFMA is issued with the weight fragment as its first operand, so the
// 32x32 result of v_mfma_i32_32x32x32_i8 holds, in lane l and register r,
//   output row    m = l % 32                      (token)
//   output column n = 8 (r / 4) + 4 (l / 32) + r % 4   (channel)
// i.e. every lane owns 4 runs of 4 consecutive output channels of one token:
// one row scale per lane and 8-/16-byte stores.
//
// Tile order: the 1-D grid is remapped so that each of the 8 XCDs (blocks are
// dealt to XCDs round-robin) owns a contiguous range of tiles, walked in
// column-major order within bands of GM tile rows: the blocks resident on
// one XCD share A rows and B columns in that XCD's L2.
//
// OCC is the number of waves per SIMD the register allocation must allow
// (OCC = 2 with 4-wave blocks keeps two blocks resident per CU, whose
// independent barriers interleave on every SIMD).
template <int BM, int BN, int BK, int WM, int WN, int S, int GM, bool DEQ, int OCC = 1>
__global__ __launch_bounds__((BM / WM) * (BN / WN) * 64)
__attribute__((amdgpu_waves_per_eu(OCC))) void gemm_i8_kernel(
    const int8_t* __restrict__ A, int64_t M, const int8_t* __restrict__ B, int64_t N, int K,
    int32_t* __restrict__ Cout, int64_t ldc, GemmEpi ep) {
  constexpr int NW = (BM / WM) * (BN / WN);
  constexpr int WAVES_N = BN / WN;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int NC = BK / 16;                     // 16-B chunks per tile row
  constexpr int RPB = 64 / NC;                    // tile rows per 1-KB load block
  constexpr int LA = BM / (RPB * NW), LB = BN / (RPB * NW), L = LA + LB;
  constexpr int NS = BK / 32;                     // MFMA k-steps per stage
  constexpr int SH = (BK == 128) ? 1 : 2;
  static_assert(LA * RPB * NW == BM && LB * RPB * NW == BN, "whole load instructions per wave");
  static_assert(S >= 2 && S <= 4, "2..4 stages");
  static_assert(BK == 64 || BK == 128, "BK");
  constexpr int STAGE = (BM + BN) * BK;
  __shared__ __attribute__((aligned(1024))) uint8_t smem[S * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int64_t m0, n0;
  {
    const int tmt = int((M + BM - 1) / BM), tnt = int((N + BN - 1) / BN);
    const int ntiles = tmt * tnt;
    int tile = blockIdx.x;
    if ((ntiles & 7) == 0) tile = (tile & 7) * (ntiles >> 3) + (tile >> 3);
    const int g = tile / (GM * tnt), r = tile - g * (GM * tnt);
    const int rows_in = (tmt - g * GM) < GM ? (tmt - g * GM) : GM;
    m0 = int64_t(g * GM + r % rows_in) * BM;
    n0 = int64_t(r / rows_in) * BN;
  }
  const int wm0 = (wave / WAVES_N) * WM, wn0 = (wave % WAVES_N) * WN;
  const int KT = K / BK;
  static_assert(4 * (3 * BN + 2 * BM) <= S * STAGE, "epilogue staging fits in LDS");

  // Per load instruction q: global row pointer (rows clamped into range) and
  // the 1-KB LDS block it fills.
  const int8_t* gsrc[L];
  int ldst[L];
#pragma unroll
  for (int q = 0; q < L; ++q) {
    const bool isA = q < LA;
    const int blk = (isA ? q : q - LA) * NW + wave;   // 1-KB block index in the A or B tile
    const int slot = blk * 64 + lane;                 // 16-B slot index
    const int row = slot / NC;
    const int c = (slot % NC) ^ ((row >> SH) & (NC - 1));
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
  // Fragment reads of k-step `s_` (0..NS-1) of the stage in buffer `buf_`.
#define HQ_READ_FRAGS(SET_, buf_, s_)                                                      \
  do {                                                                                     \
    const uint8_t* cur_ = smem + (buf_) * STAGE;                                           \
    const int c_ = 2 * (s_) + lhalf;                                                       \
    _Pragma("unroll") for (int i = 0; i < TM; ++i) af[SET_][i] =                           \
        *reinterpret_cast<const v4i*>(cur_ + swz<BK>(wm0 + i * 32 + lrow, c_));            \
    _Pragma("unroll") for (int j = 0; j < TN; ++j) bfr[SET_][j] =                          \
        *reinterpret_cast<const v4i*>(cur_ + BM * BK + swz<BK>(wn0 + j * 32 + lrow, c_));  \
  } while (0)
  // Waits until stage `kt_` has landed (later stages may still fly), then
  // joins the block.
#define HQ_WAIT_STAGE(kt_)                                                                 \
  do {                                                                                     \
    const int ahead_ = KT - 1 - (kt_);                                                     \
    if (S >= 4 && ahead_ >= 2)                                                             \
      wait_vm_lgkm0<(S >= 4 ? 2 * L : 0)>();                                               \
    else if (S >= 3 && ahead_ >= 1)                                                        \
      wait_vm_lgkm0<(S >= 3 ? L : 0)>();                                                   \
    else                                                                                   \
      wait_vm_lgkm0<0>();                                                                  \
    __builtin_amdgcn_s_barrier();                                                          \
  } while (0)

  v4i af[2][TM], bfr[2][TN];
  HQ_WAIT_STAGE(0);
  HQ_READ_FRAGS(0, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    // Buffer (kt-1) % S was fully read before the barrier that ended the
    // previous stage, so stage kt+S-1 may land there now.
    if (kt + S - 1 < KT) HQ_ISSUE_STAGE(kt + S - 1);
    const int buf = kt % S;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int cs = s & 1;
      if (s + 1 < NS) {
        if (cs == 0) HQ_READ_FRAGS(1, buf, s + 1); else HQ_READ_FRAGS(0, buf, s + 1);
      } else if (kt + 1 < KT) {
        // Last k-step: retire this stage block-wide, then fetch the first
        // fragments of the next stage before issuing this step's MFMAs.
        HQ_WAIT_STAGE(kt + 1);
        HQ_READ_FRAGS(0, (kt + 1) % S, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bfr[cs][j], af[cs][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#undef HQ_READ_FRAGS
#undef HQ_WAIT_STAGE
#undef HQ_ISSUE_STAGE

  gemm_epilogue<BM, BN, TM, TN, NW, DEQ>(acc, smem, tid, lane, m0, n0, wm0, wn0, M, N, Cout, ldc, ep);
}

}  // namespace hq
