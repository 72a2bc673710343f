// Device helpers shared by the gfx950 kernels of libhq (HIP, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// bf16 is carried as raw uint16_t bit patterns on the device side.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// float -> bf16, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Two floats -> packed bf16 pair (low half = a), one v_cvt_pk_bf16_f32.
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((v2f){a, b}, v2bf));
}

// Load 8 consecutive elements as float.
__device__ __forceinline__ void load8(const float* __restrict__ p, float v[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* __restrict__ p, float v[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = __uint_as_float(u.x << 16); v[1] = __uint_as_float(u.x & 0xFFFF0000u);
  v[2] = __uint_as_float(u.y << 16); v[3] = __uint_as_float(u.y & 0xFFFF0000u);
  v[4] = __uint_as_float(u.z << 16); v[5] = __uint_as_float(u.z & 0xFFFF0000u);
  v[6] = __uint_as_float(u.w << 16); v[7] = __uint_as_float(u.w & 0xFFFF0000u);
}

// Symmetric code of v with reciprocal scale rcp = qmax / max|v|, in the low
// byte: fma(v, rcp, 1.5 * 2^23) rounds the exact product v * rcp once, ties
// to even, onto the integer grid of [2^23, 2^24) (|v * rcp| <= qmax (1 + 2^-24),
// so no clamp is needed); the low byte is the code in two's complement.
__device__ __forceinline__ uint32_t code_bits(float v, float rcp) {
  return __float_as_uint(fmaf(v, rcp, 12582912.0f));
}
// Four codes -> one dword (byte k = code k).
__device__ __forceinline__ uint32_t pack_codes4(float a, float b, float c, float d, float rcp) {
  const uint32_t ab = __builtin_amdgcn_perm(code_bits(b, rcp), code_bits(a, rcp), 0x0c0c0400u);
  const uint32_t cd = __builtin_amdgcn_perm(code_bits(d, rcp), code_bits(c, rcp), 0x0c0c0400u);
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);
}

// Four codes as E2M3 bytes (byte k = code of the k-th value): the magnitude
// |q| = rint(|v| rcp) in 0..7 indexes the table of E2M3 encodings
// {0, 8, 16, 20, 24, 26, 28, 30} with one byte permute; the sign bit (bit 5)
// is set for negative v with q != 0, so that q = 0 is always +0.
__device__ __forceinline__ uint32_t e2m3_codes4(float a, float b, float c, float d, float rcp) {
  const uint32_t mag = pack_codes4(fabsf(a), fabsf(b), fabsf(c), fabsf(d), rcp);
  const uint32_t t = __builtin_amdgcn_perm(0x1E1C1A18u, 0x14100800u, mag);
  const uint32_t s01 = __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x0c0c0703u);
  const uint32_t s23 = __builtin_amdgcn_perm(__float_as_uint(d), __float_as_uint(c), 0x07030c0cu);
  const uint32_t nz = (t + 0x7F7F7F7Fu) & 0x80808080u;  // bit 7 of byte k: code k != 0
  return t | (((s01 | s23) & nz) >> 2);
}
// Four 6-bit values in the bytes of x -> one 24-bit little-endian string.
__device__ __forceinline__ uint32_t pack6x4(uint32_t x) {
  const uint32_t y = (x & 0x003F003Fu) | ((x >> 2) & 0x0FC00FC0u);
  return (y & 0xFFFu) | ((y >> 4) & 0xFFF000u);
}
// Byte offset of the 6-byte piece holding channels e0 .. e0+7 (e0 a
// multiple of 8) of `row` in the E2M3 layout of a d-channel code matrix with
// R-row groups: (row / R) 3 R d / 4 + (e0 / 128) 96 R + (row % R) 96 +
// 6 ((e0 % 128) / 8).
template <int R>
__device__ __forceinline__ int64_t e2m3_piece_offset(int64_t row, int d, int e0) {
  return (row / R) * (int64_t(R) * 3 / 4) * int64_t(d) + (e0 >> 7) * (96 * R) + (row % R) * 96 +
         6 * ((e0 & 127) >> 3);
}

// Stores the E2M3 codes of the 8 values v (channels e0 .. e0+7 of `row`,
// e0 a multiple of 8) at their piece of the R-row-group layout, written as a
// dword and a short at their natural alignment.
template <int R>
__device__ __forceinline__ void store_e2m3x8(uint8_t* __restrict__ codes, int64_t row, int d,
                                             int e0, const float* v, float rcp) {
  const uint32_t p0 = pack6x4(e2m3_codes4(v[0], v[1], v[2], v[3], rcp));
  const uint32_t p1 = pack6x4(e2m3_codes4(v[4], v[5], v[6], v[7], rcp));
  const uint32_t w0 = p0 | (p1 << 24), w1 = p1 >> 8;  // 48-bit piece
  uint8_t* p = codes + e2m3_piece_offset<R>(row, d, e0);
  const bool odd = e0 & 8;  // odd pieces start 2 bytes past a dword boundary
  *reinterpret_cast<uint32_t*>(p + (odd ? 2 : 0)) = odd ? __builtin_amdgcn_alignbit(w1, w0, 16) : w0;
  *reinterpret_cast<uint16_t*>(p + (odd ? 0 : 4)) = uint16_t(odd ? w0 : w1);
}

// Direct global -> LDS copy of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): the wave's 64 lanes fill 1 KB of LDS starting at
// the wave-uniform address `lds`, lane l at lds + 16 l. Completion is tracked
// by vmcnt; callers wait explicitly. The builtin exists only in the device
// pass, where it is the whole body.
__device__ __forceinline__ void lds_dma16(const void* gptr, void* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(gptr, lds, 16, 0, 0);
#endif
}

// Cross-lane exchange on the VALU (no LDS traffic). lane_xor<M>(v) returns v
// of lane (lane ^ M) for M in {1, 2, 4, 8} through DPP: quad_perm for 1 and
// 2, row_ror:8 for 8, and row_half_mirror (i ^ 7) followed by
// quad_perm[3,2,1,0] (i ^ 3) for 4.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  const int x = __float_as_int(v);
  if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
  if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
  if constexpr (M == 8) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x128, 0xF, 0xF, false));
  if constexpr (M == 4) {
    const int h = __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
    return __int_as_float(__builtin_amdgcn_mov_dpp(h, 0x1B, 0xF, 0xF, false));
  }
  static_assert(M == 1 || M == 2 || M == 4 || M == 8, "lane_xor distance");
  return v;
}

// (value of the lower lane, value of the upper lane) of the pair
// {lane, lane ^ M} for M in {16, 32}: gfx950 v_permlane16/32_swap with both
// operands equal to v leaves the lower-half value in [0] and the upper-half
// value in [1], in both lanes of the pair.
template <int M>
__device__ __forceinline__ void lane_pair(float v, float* lo, float* hi) {
  const unsigned x = __float_as_uint(v);
  if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    *lo = __uint_as_float(r[0]);
    *hi = __uint_as_float(r[1]);
  } else {
    static_assert(M == 32, "lane_pair distance");
    const auto r = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    *lo = __uint_as_float(r[0]);
    *hi = __uint_as_float(r[1]);
  }
}

// One Walsh-Hadamard butterfly across lanes at distance M: the lower lane of
// each pair keeps a_lo + a_hi, the upper lane a_lo - a_hi. `sg` is +1 on
// lower lanes and -1 on upper lanes.
template <int M>
__device__ __forceinline__ float butterfly(float v, float sg) {
  if constexpr (M <= 8) {
    return fmaf(sg, v, lane_xor<M>(v));
  } else {
    float lo, hi;
    lane_pair<M>(v, &lo, &hi);
    return fmaf(sg, hi, lo);
  }
}

// All-reduce over aligned groups of G lanes; every lane of a group ends with
// the bit-identical result (each pairwise step adds the same two operands).
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  if constexpr (G >= 2) v += lane_xor<1>(v);
  if constexpr (G >= 4) v += lane_xor<2>(v);
  if constexpr (G >= 8) v += lane_xor<4>(v);
  if constexpr (G >= 16) v += lane_xor<8>(v);
  if constexpr (G >= 32) { float lo, hi; lane_pair<16>(v, &lo, &hi); v = lo + hi; }
  if constexpr (G >= 64) { float lo, hi; lane_pair<32>(v, &lo, &hi); v = lo + hi; }
  return v;
}
template <int G>
__device__ __forceinline__ float group_max(float v) {
  if constexpr (G >= 2) v = fmaxf(v, lane_xor<1>(v));
  if constexpr (G >= 4) v = fmaxf(v, lane_xor<2>(v));
  if constexpr (G >= 8) v = fmaxf(v, lane_xor<4>(v));
  if constexpr (G >= 16) v = fmaxf(v, lane_xor<8>(v));
  if constexpr (G >= 32) { float lo, hi; lane_pair<16>(v, &lo, &hi); v = fmaxf(lo, hi); }
  if constexpr (G >= 64) { float lo, hi; lane_pair<32>(v, &lo, &hi); v = fmaxf(lo, hi); }
  return v;
}

}  // namespace hq
