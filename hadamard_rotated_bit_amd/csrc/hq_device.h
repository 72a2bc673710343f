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

// float -> bf16, round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
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

// Round-half-even to an integer held in the low byte: adding 1.5 * 2^23 puts
// rint(v) (|v| < 2^22) in the low mantissa bits, two's complement mod 2^8.
__device__ __forceinline__ uint32_t rne_byte(float v) {
  return __float_as_uint(v + 12582912.0f) & 0xFFu;
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

// Butterfly partner across lanes: value of lane (lane ^ mask).
__device__ __forceinline__ float xor_shfl(float v, int mask) { return __shfl_xor(v, mask, 64); }

}  // namespace hq
