// Internal launcher interface between the C ABI (hq_abi.cpp) and the kernels.
// Launchers enqueue on `stream` and return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "hq_gemm_types.h"

namespace hq {

// Sets the calling thread's error text (what hq_last_error returns) and
// returns `code`; for entry points defined outside hq_abi.cpp.
int set_error(int code, const char* msg);

// GEMM macro tile sizes; d_out is padded to a multiple of GEMM_BN in the
// prepared blob and T to a multiple of GEMM_BM in the workspace.
constexpr int GEMM_BM = 256;
constexpr int GEMM_BN = 256;

// Row-transform geometry: G lanes per row, C chunks of 8*G channels per lane.
struct RowGeom {
  int G, C;
};
bool row_geometry(int d_in, RowGeom* g);

enum RowMode { ROW_ACT = 0, ROW_WEIGHT = 1, ROW_EXPORT = 2 };

// Code storage (the C ABI's hq_code_format_t): int8 bytes, or E2M3 fp6 in
// groups of R = F6_GROUP rows (group g of rows at 3 R d g / 4 bytes; 128-code
// slice s of row R g + i at byte 96 R s + 96 i inside it; code k of the
// slice at bits 6k).
enum CodeFmt { CODES_I8 = 0, CODES_E2M3 = 1 };
inline size_t code_bytes(int fmt, int64_t rows, int d) {
  if (fmt == CODES_E2M3)
    return size_t((rows + F6_GROUP - 1) / F6_GROUP) * (size_t(F6_GROUP) * 3 / 4) * size_t(d);
  return size_t(rows) * size_t(d);
}

struct RowArgs {
  const void* in;         // [rows, d] f32 or bf16
  int in_bf16;
  int64_t rows;
  int d;
  const float* scale;     // per-channel multiplier (1/sigma or sigma); NULL = ones
  const float* chan_mean; // per-channel value subtracted before the multiplier
                          // (per-channel centring); NULL = none. Needs scale
                          // (ones for no smoothing).
  int log2b;
  int center;
  float qmax;
  uint8_t* codes;         // rows x d codes in code_fmt (ACT, WEIGHT)
  int code_fmt;           // CodeFmt
  float* out_s;           // [rows] dequant scale  (ACT, WEIGHT); with group > 0
                          // [d / group, s_ld], one scale per row and group
  int group;              // 0: one scale per row; 64: one per 64-channel group
  int64_t s_ld;           // row stride of out_s between groups (group > 0)
  float* out_aux;         // [rows] mu (ACT, EXPORT) or c (WEIGHT); NULL = not written
  float* out_xt;          // [rows, d] f32         (EXPORT)
  int mode;
};
hipError_t launch_row_transform(const RowArgs& a, hipStream_t s);
// The fast kernel for blocks of at least 8 G channels; hipErrorNotSupported
// when the geometry has no instance (the general kernel then runs).
hipError_t launch_row_fast(const RowArgs& a, const RowGeom& g, hipStream_t s);
// The fast row transform (activation mode) and the rank-r down projection
// U [rows, r] = in . (l1_hi + l1_lo)^T in one launch; act_lr_applies says
// whether the geometry has this form (bf16 input, G = 64 with C = 5 or 6,
// r = 16 or 32, blocks of >= 512 channels, no per-channel means or groups),
// launch_act_lr returns hipErrorNotSupported where it has not.
bool act_lr_applies(const RowArgs& a, const RowGeom& g, int r);
hipError_t launch_act_lr(const RowArgs& a, const RowGeom& g, int r, const uint16_t* l1_hi,
                         const uint16_t* l1_lo, float* U, hipStream_t s);

// absmax[i] = max over rows of |in[r, i]| ; absmax zeroed by the launcher.
hipError_t launch_col_absmax(const void* in, int in_bf16, int64_t rows, int d, float* absmax,
                             hipStream_t s);
// sigma[i] = max(ax_i, eps)^alpha / max(sigma[i], eps)^(1 - alpha) in place.
hipError_t launch_sigma_finish(const float* ax, float alpha, float eps, int d, float* sigma,
                               hipStream_t s);

// Fill n floats / bytes.
hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s);
hipError_t launch_fill_u8(uint8_t* p, uint8_t v, size_t n, hipStream_t s);
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t s);
hipError_t launch_reciprocal(const float* src, float* dst, int n, hipStream_t s);
// Write a small POD header (<= 256 bytes) to device memory.
hipError_t launch_write_header(const void* host_hdr, size_t bytes, void* dst, hipStream_t s);

// Low-rank factors: l1 [d, r] -> (l1 / sigma)^T split into bf16 hi/lo [r, d];
// l2 [r, n] -> l2^T split into bf16 hi/lo [n_pad, r] (rows >= n zero).
hipError_t launch_prep_l1(const void* l1, int bf16, const float* sigma_inv, int d, int r,
                          uint16_t* hi, uint16_t* lo, hipStream_t s);
hipError_t launch_prep_l2(const void* l2, int bf16, int r, int n, int n_pad, uint16_t* hi,
                          uint16_t* lo, hipStream_t s);

// U [rows, r] = x [rows, d] . (l1_hi + l1_lo)^T  (bf16 MFMA, fp32 accumulate).
hipError_t launch_lowrank_down(const void* x, int x_bf16, int64_t rows, int d, int r,
                               const uint16_t* l1_hi, const uint16_t* l1_lo, float* U,
                               hipStream_t s);
// The same U in two passes: per slice of d, products for 128 rows per block
// with the slice of l1 shared in LDS, into part [slices, rows, r]; then the
// slices summed in order. lowrank_slices(d, r, rows) is the slice count
// (4, 6 or 8, chosen for the row count; the partition the one-pass kernel
// gives its waves, so U is bit-identical), or 0 where the split form does
// not apply.
int lowrank_slices(int d, int r, int64_t rows);
hipError_t launch_lowrank_split(const void* x, int x_bf16, int64_t rows, int d, int r,
                                const uint16_t* l1_hi, const uint16_t* l1_lo, float* part,
                                float* U, hipStream_t s);

// Per-channel centring (center = 2): partial column sums over chunks of
// CENTER_RPC rows, then mean [d]; partial holds center_chunks(rows) x d floats.
constexpr int CENTER_RPC = 64;
int center_chunks(int64_t rows);
hipError_t launch_channel_mean(const void* x, int x_bf16, int64_t rows, int d, float* partial,
                               float* mean, hipStream_t s);
// out [n_pad] = bias + weight [n, d] . mean (rows n..n_pad-1: bias).
hipError_t launch_bias_gemv(const void* weight, int w_bf16, const float* mean, const float* bias,
                            int n, int n_pad, int d, float* out, hipStream_t s);


// acc = A [M, K] . B [N, K]^T ; epilogue: int32 store to acc_out (ld = ldc) when
// epi == NULL, else the dequant epilogue. Loads of rows past M / N are
// clamped to the last row.
hipError_t launch_gemm(const int8_t* A, int64_t M, const int8_t* B, int64_t N, int K,
                       int32_t* acc_out, int64_t ldc, const GemmEpi* epi, hipStream_t s);
// The same product on E2M3 codes (CODES_E2M3 layout, M and N rows; K a
// multiple of 128) with the FP6 MFMA; rows past M / N in their last row
// group must be readable (their results are discarded).
// Group-wise FP6 GEMM with the dequant epilogue: 64-code groups, s_xg [K/64,
// ld_sx] and s_wg [K/64, ld_sw] one scale per row / column and group; the
// epilogue adds b + mu c (+ low rank) to the group-scaled sums. K % 128 == 0.
hipError_t launch_gemm_f6g(const uint8_t* A, int64_t M, const uint8_t* B, int64_t N, int K,
                           const float* s_xg, int64_t ld_sx, const float* s_wg, int64_t ld_sw,
                           const GemmEpi* epi, hipStream_t s);
hipError_t launch_gemm_f6(const uint8_t* A, int64_t M, const uint8_t* B, int64_t N, int K,
                          int32_t* acc_out, int64_t ldc, const GemmEpi* epi, hipStream_t s);

// Integer-only DH / WH layers with integer requantisation.
constexpr int WH_MAX_BLOCK = 256;       // largest output-side Hadamard order
constexpr int WH_SHIFT_MAX = 48;        // largest shared requantisation shift
constexpr int WH_MULT_MAX = 32767;      // multipliers fit a positive 16-bit integer
constexpr int WH_BIAS_MAX = 1 << 27;    // bias codes saturate here (exact float64 requant)
// wbar [acc_rows, d_in] f32 = H_m (blocks of m output channels) . [weight; 0]
// (weight [d_out, d_in]; rows d_out .. acc_rows - 1 of a padded order are zero).
hipError_t launch_wh_weight(const void* w, int w_bf16, int d_out, int acc_rows, int d_in, int m,
                            float* wbar, hipStream_t s);
// out [rows, width] f32 = [w 0] (w [rows, d_in], zeros in columns d_in ..).
hipError_t launch_pad_rows(const void* w, int w_bf16, int64_t rows, int d_in, int width,
                           float* out, hipStream_t s);
// The transition after an integer layer: the transform before the
// activation (m), the activation (hq_int_act), the transform after it (post),
// and the prepared constants (bias codes, per-channel multipliers, the shift;
// for SiLU/GELU also the table over z + 127, M_in and n_in).
struct IntTransition {
  int m, post, act;
  int keep;   // channels kept after H~_m (the layer's d_out)
  const int32_t* b_int;
  const int32_t* mult;
  const int32_t* shift;
  const int8_t* lut;
  const int32_t* mult_in;
  const int32_t* shift_in;
};
// b_int, mult [d_out_pad] and shift [1] from bias [d_out] (or NULL; b-bar =
// b H over blocks of bias_block channels) and s_w [d_out]. Identity / ReLU:
// rho = s_x s_w / (sqrt(m post) s_y). SiLU / GELU: rho = s_x s_w / (sqrt(m)
// s_z), the table lut [256] (entry z + 127 = clamp(round(phi(s_z z) / s_u));
// entry 255 = 0), M_in and n_in from s_u / (sqrt(post) s_y).
hipError_t launch_int_constants(const float* bias, int n_bias, const float* s_w, int acc_w,
                                int d_out_pad, int m, int post, int act, int bias_block,
                                float s_x, float s_y, float s_z, float s_u, int32_t* b_int,
                                int32_t* mult, int32_t* shift, int8_t* lut, int32_t* mult_in,
                                int32_t* shift_in, hipStream_t s);
// The integer GEMM and the transition's requantisation in one kernel
// (d_out % 256 == 0): y [T, d_out] from x [T, d_in] int8 and w [>= d_out,
// d_in] int8; the int32 products stay on the chip.
hipError_t launch_int_fused(const int8_t* x, int64_t T, int d_in, const int8_t* w, int d_out,
                            const IntTransition& tr, int8_t* y, hipStream_t s);
// y [T, ldy] int8 (out_w channels) from acc [T, ldc] (acc_w channels, without
// the bias codes): the transition's requantisation.
hipError_t launch_int_requant(const int32_t* acc, int64_t ldc, int64_t T, int acc_w, int out_w,
                              const IntTransition& tr, int8_t* y, int64_t ldy, hipStream_t s);

}  // namespace hq
