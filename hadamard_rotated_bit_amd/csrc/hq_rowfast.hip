// Fast row transform of libhq for the common geometry: the Hadamard block
// covers at least the 8 G channels spread over a row's lanes, so every
// butterfly stage on the register and lane bits is taken, and the NX stages
// on chunk-index bits are a compile-time count. (Smaller blocks use the
// general kernel in hq_act.hip.)
//
// Same arithmetic per row as the general kernel (HadaNorm Eq. (1) activation
// side, HaTQ Sec. III-A Eq. (3) quantiser), with these differences in how
// the lanes carry it out:
//  * Cross-lane butterflies are one v_fmac_f32_dpp each where a DPP pattern
//    reaches the partner (v += g * v[partner], g = +1 on the lower and -1 on
//    the upper lane of a pair): lane ^ 1 and lane ^ 2 (quad permutes),
//    lane ^ 8 (row rotation by 8) and lane ^ 7 (half-row mirror); distance
//    16 uses ds_swizzle plus one fma, distance 32 v_permlane32_swap. The
//    xor-7 stage runs first, on channel bit 5 (lane bit 2): butterflies over
//    the masks 7, 1, 2 (then 8, 16, 32) give the Sylvester transform with its
//    outputs permuted, lane t holding channel pi(t) = t with bit 2 flipped
//    when bits 0 and 1 differ, so results are stored at pi(t). The upper lane
//    of a pair holds the negated difference: after all stages lane t stores
//    sigma_t times the transformed value, with sigma_t = (-1)^popcount(t &
//    NEG) (NEG = the lane bits done in this form), negated again on lanes
//    with t mod 8 = 5 or 6 (the xor-7 stage's pairing). The mean is
//    subtracted as sigma_t * mu and the quantiser uses sigma_t * (qmax /
//    absmax): every code and scale is the same as with unsigned storage, bit
//    for bit.
//  * E2M3 codes come from v_cvt_scalef32_2xpk16_fp6_f32 on the integer codes
//    rint(x * qmax / absmax) (formed as fma(x, r, 1.5 2^23) - 1.5 2^23, one
//    rounding of the exact product), 32 codes per instruction; the
//    instruction interleaves its two 16-value halves (field 2i holds x[i],
//    field 2i+1 holds y[i]), so four chunks of 8 channels are fed in that
//    order and come out as four 48-bit pieces.
//  * No runtime stage tests, so the butterflies run in place.
//  * The row sum (for the mean, and c for weights) is taken from the closed
//    form B * sum of the blocks' first inputs instead of summing every
//    output.
//  * The per-channel multipliers and means are staged once per block in LDS
//    (template mode P: none, multipliers, multipliers and means).
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {

typedef unsigned v6u __attribute__((ext_vector_type(6)));

// v[i] += v[lane ^ M][i] * g for the 8 registers of a chunk, one DPP fma
// each. The leading s_nop covers the DPP read-after-VALU-write hazard for
// the first instruction; the others read registers written before the block.
#define HQ_DPP_FMAC8(CTRL)                                                         \
  asm("s_nop 1\n\t"                                                                \
      "v_fmac_f32_dpp %0, %0, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
      "v_fmac_f32_dpp %1, %1, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
      "v_fmac_f32_dpp %2, %2, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
      "v_fmac_f32_dpp %3, %3, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
      "v_fmac_f32_dpp %4, %4, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
      "v_fmac_f32_dpp %5, %5, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
      "v_fmac_f32_dpp %6, %6, %8 " CTRL " row_mask:0xf bank_mask:0xf\n\t"          \
      "v_fmac_f32_dpp %7, %7, %8 " CTRL " row_mask:0xf bank_mask:0xf"              \
      : "+v"(v[0]), "+v"(v[1]), "+v"(v[2]), "+v"(v[3]), "+v"(v[4]), "+v"(v[5]),   \
        "+v"(v[6]), "+v"(v[7])                                                     \
      : "v"(g))

// One cross-lane butterfly stage at lane distance M on a chunk of 8 values.
// M = 1, 2, 4, 8, 16: negating form v + g v[lane ^ M]; M = 32: true form
// lo + g hi from the permlane32 swap.
template <int M>
__device__ __forceinline__ void xstage8(float* v, float g) {
  if constexpr (M == 1) {
    HQ_DPP_FMAC8("quad_perm:[1,0,3,2]");
  } else if constexpr (M == 2) {
    HQ_DPP_FMAC8("quad_perm:[2,3,0,1]");
  } else if constexpr (M == 8) {
    HQ_DPP_FMAC8("row_ror:8");
  } else if constexpr (M == 7) {
    HQ_DPP_FMAC8("row_half_mirror");   // lane ^ 7 inside each 8-lane half row
  } else if constexpr (M == 4 || M == 16) {
    // ds_swizzle bitmask mode on 32-lane groups: lane reads lane ^ M.
    constexpr int pat = 0x1F | (M << 10);
    float p[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      p[j] = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v[j]), pat));
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = fmaf(p[j], g, v[j]);
  } else {
    static_assert(M == 32, "lane distance");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      float lo, hi;
      lane_pair<32>(v[j], &lo, &hi);
      v[j] = fmaf(g, hi, lo);
    }
  }
}
#undef HQ_DPP_FMAC8

// One 48-bit piece (w0 = bits 0..31, w1 = bits 32..47) at p; p is 4-byte
// aligned (odd = false) or 2 bytes past (odd = true).
__device__ __forceinline__ void store_piece48(uint8_t* p, uint32_t w0, uint32_t w1, bool odd) {
  *reinterpret_cast<uint32_t*>(p + (odd ? 2 : 0)) = odd ? __builtin_amdgcn_alignbit(w1, w0, 16) : w0;
  *reinterpret_cast<uint16_t*>(p + (odd ? 0 : 4)) = uint16_t(odd ? w0 : w1);
}

// Everything after a row's loads: means and multipliers, the butterflies,
// the centring and the quantiser, for the row `row` whose lane-t chunks are
// in v. lpar holds the block's multipliers (P >= 1) and, from float4 MO on,
// its means (P = 2).
template <int G, int C, int NX, int P, int MO>
__device__ __forceinline__ void row_fast_body(const RowArgs& a, float inv_sqrt_b, int t,
                                              int64_t row, bool valid, float* v,
                                              const float4* lpar) {
  constexpr int E = 8 * C;
  constexpr int NEG = (G >= 32) ? 31 : 15;  // lane bits done in negating form
  const int d = a.d;
  const float g1 = (t & 1) ? -1.0f : 1.0f, g2 = (t & 2) ? -1.0f : 1.0f;
  const float g4 = (t & 4) ? -1.0f : 1.0f, g8 = (t & 8) ? -1.0f : 1.0f;
  const float g16 = (t & 16) ? -1.0f : 1.0f, g32 = (t & 32) ? -1.0f : 1.0f;
  const float sgn = ((__builtin_popcount(t & NEG) & 1) ? -1.0f : 1.0f) *
                    (((t & 7) == 5 || (t & 7) == 6) ? -1.0f : 1.0f);
  // channel position of the lane's transformed values (see the file comment)
  const int pt = t ^ (((t ^ (t >> 1)) & 1) << 2);

  // Row sum of the unnormalised transform: every row of a Sylvester H~_B
  // but the first sums to zero, so the sum over a block's outputs is B times
  // its first input; lane 0 of a row holds the first input of the blocks
  // starting at its chunks c = 0 mod 2^NX.
  float s0 = 0.0f;
#pragma unroll
  for (int c = 0; c < C; ++c) {
    float* vc = &v[c * 8];
    if constexpr (P == 2) {
      const float4 m0 = lpar[MO + c * 2 * G + 2 * t], m1 = lpar[MO + c * 2 * G + 2 * t + 1];
      vc[0] -= m0.x; vc[1] -= m0.y; vc[2] -= m0.z; vc[3] -= m0.w;
      vc[4] -= m1.x; vc[5] -= m1.y; vc[6] -= m1.z; vc[7] -= m1.w;
    }
    if constexpr (P > 0) {
      const float4 s0_ = lpar[c * 2 * G + 2 * t], s1_ = lpar[c * 2 * G + 2 * t + 1];
      vc[0] *= s0_.x; vc[1] *= s0_.y; vc[2] *= s0_.z; vc[3] *= s0_.w;
      vc[4] *= s1_.x; vc[5] *= s1_.y; vc[6] *= s1_.z; vc[7] *= s1_.w;
    }
    if ((c & ((1 << NX) - 1)) == 0) s0 += vc[0];
    // channel bits 0..2, in registers
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if (!(e & h)) {
          const float x = vc[e], y = vc[e + h];
          vc[e] = x + y;
          vc[e + h] = x - y;
        }
      }
    }
    // channel bits 3 .. 3 + log2 G - 1, across lanes
    xstage8<7>(vc, g4);
    xstage8<1>(vc, g1);
    xstage8<2>(vc, g2);
    xstage8<8>(vc, g8);
    if constexpr (G >= 32) xstage8<16>(vc, g16);
    if constexpr (G >= 64) xstage8<32>(vc, g32);
  }
  // channel bits above: chunk index bits 0 .. NX-1, in registers
#pragma unroll
  for (int b = 0; b < NX; ++b) {
    const int h = 1 << b;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      if (!(c & h)) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = v[c * 8 + j], y = v[(c + h) * 8 + j];
          v[c * 8 + j] = x + y;
          v[(c + h) * 8 + j] = x - y;
        }
      }
    }
  }

  const float sum = float(1 << a.log2b) * group_sum<G>(t == 0 ? s0 : 0.0f);

  const bool weight = a.mode == ROW_WEIGHT;
  const float mu = (!weight && a.center) ? sum / float(d) : 0.0f;
  const float smu = sgn * mu;
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] -= smu;
    amax = fmaxf(amax, fabsf(v[e]));
  }
  if (a.mode == ROW_EXPORT) {
    if (valid) {
      const float sc = sgn * inv_sqrt_b;
      float* o = a.out_xt + row * d + pt * 8;
#pragma unroll
      for (int c = 0; c < C; ++c) {
        const float* vc = &v[c * 8];
        reinterpret_cast<float4*>(o + c * 8 * G)[0] =
            make_float4(vc[0] * sc, vc[1] * sc, vc[2] * sc, vc[3] * sc);
        reinterpret_cast<float4*>(o + c * 8 * G)[1] =
            make_float4(vc[4] * sc, vc[5] * sc, vc[6] * sc, vc[7] * sc);
      }
      if (t == 0 && a.out_aux) a.out_aux[row] = mu * inv_sqrt_b;
    }
    return;
  }
  amax = group_max<G>(amax);
  const float rs = sgn * (amax > 0.0f ? a.qmax / amax : 0.0f);
  if (!valid) return;
  if (a.code_fmt == CODES_E2M3) {
    constexpr float MAGIC = 12582912.0f;  // 1.5 * 2^23
    const bool odd = pt & 1;
    uint8_t* rb = a.codes + e2m3_piece_offset<F6_GROUP>(row, d, 0);
#pragma unroll
    for (int c0 = 0; c0 < C; c0 += 4) {
      v16f x, y;
#pragma unroll
      for (int m = 0; m < 4; ++m)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float q = (c0 + m < C) ? fmaf(v[(c0 + m) * 8 + j], rs, MAGIC) - MAGIC : 0.0f;
          if (j & 1) y[4 * m + j / 2] = q; else x[4 * m + j / 2] = q;
        }
      const v6u p = __builtin_amdgcn_cvt_scalef32_2xpk16_fp6_f32(x, y, 1.0f);
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (c0 + m >= C) break;
        const int e0 = (c0 + m) * 8 * G + pt * 8;
        uint8_t* dst = rb + (e0 >> 7) * (96 * F6_GROUP) + 6 * ((e0 & 127) >> 3);
        uint32_t w0, w1;
        if (m == 0) { w0 = p[0]; w1 = p[1] & 0xFFFFu; }
        else if (m == 1) { w0 = __builtin_amdgcn_alignbit(p[2], p[1], 16); w1 = p[2] >> 16; }
        else if (m == 2) { w0 = p[3]; w1 = p[4] & 0xFFFFu; }
        else { w0 = __builtin_amdgcn_alignbit(p[5], p[4], 16); w1 = p[5] >> 16; }
        store_piece48(dst, w0, w1, odd);
      }
    }
  } else {
    const int64_t base = row * d + pt * 8;
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float* vc = &v[c * 8];
      *reinterpret_cast<uint2*>(a.codes + base + c * 8 * G) =
          make_uint2(pack_codes4(vc[0], vc[1], vc[2], vc[3], rs),
                     pack_codes4(vc[4], vc[5], vc[6], vc[7], rs));
    }
  }
  if (t == 0) {
    a.out_s[row] = amax * inv_sqrt_b / a.qmax;
    if (a.out_aux) a.out_aux[row] = (weight ? sum : mu) * inv_sqrt_b;
  }
}


template <typename TIn, int G, int C, int NX, int P>
__global__ __launch_bounds__(256) void row_fast_kernel(RowArgs a, float inv_sqrt_b) {
  constexpr int LOG2G = (G == 16) ? 4 : (G == 32) ? 5 : 6;
  constexpr int E = 8 * C;
  constexpr int RPW = 64 / G;
  static_assert((C >> NX) << NX == C, "chunk stages pair whole chunks");
  const int lane = threadIdx.x & 63;
  const int t = lane & (G - 1);
  const int64_t row = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RPW + lane / G;
  const bool valid = row < a.rows;
  const int64_t r = valid ? row : a.rows - 1;
  const int d = a.d;
  const TIn* src = static_cast<const TIn*>(a.in) + r * d + t * 8;

  // The channel multipliers (P >= 1) and means (P = 2) are the same for
  // every row: the block stages them once in LDS and each lane reads its 8
  // per chunk there, so they hold no per-lane registers across the row and
  // take no slots in the vector memory queue behind the row. Their loads go
  // first (loads retire in issue order, so issued after the row they would
  // wait for the whole row); lanes past the end repeat the last float4, so
  // no load or store is conditional.
  constexpr int NV4 = 2 * C * G;                // float4 per vector (d / 4)
  constexpr int PV = (NV4 + 255) / 256;         // per thread
  constexpr int NP = P == 2 ? 2 : 1;
  __shared__ float4 lpar[P == 0 ? 1 : NP * PV * 256];
  float v[E];
  if constexpr (P > 0) {
    const int tid = threadIdx.x;
    float4 pv[NP][PV];
#pragma unroll
    for (int k = 0; k < PV; ++k) {
      const int i = k * 256 + tid < NV4 ? k * 256 + tid : NV4 - 1;
      pv[0][k] = reinterpret_cast<const float4*>(a.scale)[i];
      if constexpr (P == 2) pv[1][k] = reinterpret_cast<const float4*>(a.chan_mean)[i];
    }
#pragma unroll
    for (int c = 0; c < C; ++c) load8(src + c * 8 * G, &v[c * 8]);
#pragma unroll
    for (int q = 0; q < NP; ++q)
#pragma unroll
      for (int k = 0; k < PV; ++k) lpar[q * PV * 256 + k * 256 + tid] = pv[q][k];
    __syncthreads();
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) load8(src + c * 8 * G, &v[c * 8]);
  }

  row_fast_body<G, C, NX, P, PV * 256>(a, inv_sqrt_b, t, row, valid, v, lpar);
}

// Instantiated geometries: the (G, C) pairs row_geometry picks for the
// supported widths, each with every chunk-stage count its block sizes need.
template <typename TIn, int G, int C>
static hipError_t launch_fast_gc(const RowArgs& a, int nx, dim3 grid, float isb, hipStream_t s) {
  switch (nx) {
#define HQ_NX(N)                                                                          \
  case N:                                                                                 \
    if constexpr (((C >> N) << N) == C) {                                                 \
      if (a.chan_mean)                                                                    \
        hipLaunchKernelGGL((row_fast_kernel<TIn, G, C, N, 2>), grid, dim3(256), 0, s, a, isb); \
      else if (a.scale)                                                                   \
        hipLaunchKernelGGL((row_fast_kernel<TIn, G, C, N, 1>), grid, dim3(256), 0, s, a, isb); \
      else                                                                                \
        hipLaunchKernelGGL((row_fast_kernel<TIn, G, C, N, 0>), grid, dim3(256), 0, s, a, isb); \
      return hipGetLastError();                                                           \
    }                                                                                     \
    break;
    HQ_NX(0) HQ_NX(1) HQ_NX(2) HQ_NX(3) HQ_NX(4)
#undef HQ_NX
    default:
      break;
  }
  return hipErrorNotSupported;
}

// (G, C) pairs that row_geometry can return for a supported d_in.
template <int G, int C>
constexpr bool reachable() {
  if (G == 16) return C <= 8 || (C % 2 == 1);
  if (G == 32) return (C >= 5 && C <= 8) || (C >= 9 && C % 2 == 1);
  return C >= 5;
}

template <typename TIn, int G>
static hipError_t launch_fast_g(const RowArgs& a, int C, int nx, hipStream_t s) {
  const int rpw = 64 / G;
  const int64_t blocks = (a.rows + 4 * rpw - 1) / (4 * rpw);
  const float isb = 1.0f / sqrtf(float(1 << a.log2b));
  const dim3 grid{unsigned(blocks)};
  switch (C) {
#define HQ_C(CC)                                                  \
  case CC:                                                        \
    if constexpr (reachable<G, CC>()) return launch_fast_gc<TIn, G, CC>(a, nx, grid, isb, s); \
    return hipErrorNotSupported;
    HQ_C(1) HQ_C(2) HQ_C(3) HQ_C(4) HQ_C(5) HQ_C(6) HQ_C(7) HQ_C(8)
    HQ_C(9) HQ_C(10) HQ_C(11) HQ_C(12) HQ_C(13) HQ_C(14) HQ_C(15) HQ_C(16)
#undef HQ_C
    default:
      return hipErrorNotSupported;
  }
}

hipError_t launch_row_fast(const RowArgs& a, const RowGeom& g, hipStream_t s) {
  if (a.chan_mean && !a.scale) return hipErrorInvalidValue;
  if (a.group) return hipErrorNotSupported;  // group-wise scales: general kernel
  const int log2g = g.G == 16 ? 4 : g.G == 32 ? 5 : 6;
  const int nx = a.log2b - 3 - log2g;
  if (nx < 0 || (1 << nx) > g.C) return hipErrorNotSupported;
  if (a.in_bf16) {
    if (g.G == 16) return launch_fast_g<uint16_t, 16>(a, g.C, nx, s);
    if (g.G == 32) return launch_fast_g<uint16_t, 32>(a, g.C, nx, s);
    return launch_fast_g<uint16_t, 64>(a, g.C, nx, s);
  }
  if (g.G == 16) return launch_fast_g<float, 16>(a, g.C, nx, s);
  if (g.G == 32) return launch_fast_g<float, 32>(a, g.C, nx, s);
  return launch_fast_g<float, 64>(a, g.C, nx, s);
}

// Two 16-byte LDS reads that wait for their own results. Written as inline
// asm so that the compiler, which cannot tell these addresses from the
// targets of the LDS DMA still in flight, does not put a vmcnt(0) in front
// of them (that would drain the loads issued for the next phases).
__device__ __forceinline__ void lds_read2_b128(const uint4* p0, const uint4* p1, v4i& d0,
                                               v4i& d1) {
  const uint32_t a0 = uint32_t(reinterpret_cast<uintptr_t>(p0));
  const uint32_t a1 = uint32_t(reinterpret_cast<uintptr_t>(p1));
  asm volatile(
      "ds_read_b128 %0, %2\n"
      "ds_read_b128 %1, %3\n"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(d0), "=&v"(d1)
      : "v"(a0), "v"(a1)
      : "memory");
}

// The activation stage with the rank-r down projection in one launch, for
// bf16 input with 64 lanes per row: U = X (diag(1/sigma) L1) of the data-free
// int4 blog's low-rank branch ("Hadamard rotation: the int4 improvement",
// steps 3-4; "How it is applied here": the branch takes the smoothed input
// inside the activation pass) beside the row transform. sigma is folded into
// the prepared L1 (bf16 hi + lo, rank-major), so the branch multiplies the
// bf16 input itself, exact as an MFMA operand.
//
// Blocks below npb are projection blocks: 64 rows of U each, complete (no
// slice products to add afterwards, so no second launch). Wave w takes rows
// 16 (w % 4) .. + 15 and one half of d (w / 4); the halves advance in 24
// (d = 3072) or 20 (d = 2560) phases of 64 channels. Every load runs three
// phases ahead: a phase's L1 slices (both halves, hi and lo: 16 KB for rank
// 32) go straight from L2 into one of four LDS buffers by
// global_load_lds_dwordx4, with the chunks of rank row n rotated by
// (n / 2) mod 8 (the 16 lanes of an operand read hit 16 distinct bank
// positions), and its X operands into one of four register sets. A phase
// waits for its own loads only (an explicit vmcnt that leaves the next two
// phases' loads in flight) and meets the other waves at a bare s_barrier.
// Each 32-channel step is two v_mfma_f32_16x16x32_bf16 per 16 ranks (hi,
// then lo), and the two halves are added in a fixed order at the end. The
// other blocks run the row transform, eight rows per block. Projection
// blocks have the lowest indices, so they start first and run beside the
// row blocks, which are bound by their butterflies rather than by memory;
// both kinds fit two blocks per CU (at most 64 KB of LDS and 128 VGPRs).
constexpr int AL_ROWS = 64;   // rows of U per projection block
constexpr int AL_PH = 64;     // channels per phase and half of d
constexpr int AL_NB = 4;      // LDS buffers and X register sets (loads NB - 1 phases ahead)

template <int C, int NX, int P, int NT>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(4))) void act_lr_kernel(
    RowArgs a, float inv_sqrt_b, const uint16_t* __restrict__ l1hi,
    const uint16_t* __restrict__ l1lo, float* __restrict__ U, int npb) {
  constexpr int G = 64, E = 8 * C, R = 16 * NT;
  constexpr int D = 8 * G * C;              // channels of a row
  constexpr int DH = D / 2;                 // channels per half
  constexpr int NPH = DH / AL_PH;           // phases
  constexpr int CH = AL_PH / 8;             // 16-byte chunks of a rank row per phase
  constexpr int NV4 = 2 * C * G;            // float4 of multipliers
  constexpr int PV = (NV4 + 511) / 512;
  constexpr int LDS_LR = AL_NB * 4 * R * CH; // uint4 of the slice buffers
  constexpr int LDS_ROW = P == 0 ? 1 : PV * 512;
  static_assert(NPH * AL_PH == DH && R % 8 == 0, "whole phases and fills");
  static_assert((C >> NX) << NX == C, "chunk stages pair whole chunks");
  __shared__ uint4 lds[LDS_LR > LDS_ROW ? LDS_LR : LDS_ROW];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;

  if (int(blockIdx.x) < npb) {
    const int rg = w & 3, kh = w >> 2;
    const int kq = 8 * (lane >> 4), nl = lane & 15;
    const int64_t rbase = int64_t(blockIdx.x) * AL_ROWS + 16 * rg;
    const int64_t xrow = rbase + nl < a.rows ? rbase + nl : a.rows - 1;
    const uint16_t* const xp = static_cast<const uint16_t*>(a.in) + xrow * D + kh * DH + kq;
    // Every load runs NB - 1 phases ahead: a phase's slices go straight to
    // one of NB LDS buffers (global_load_lds_dwordx4, 1 KB per wave
    // instruction), its X operands into one of NB register sets. Slot s of
    // a buffer holds chunk (s % CH) ^ ((n / 2) % CH) of rank row
    // n = (s / CH) % R of slice s / (CH R) = 2 half + (0 hi, 1 lo), so the
    // 16 lanes of an operand read (16 rank rows, one chunk) hit 16 distinct
    // bank positions. Wave w fills units w UW .. w UW + UW - 1.
    static_assert(CH == 8, "rotation over 8 chunks per rank row");
    constexpr int UW = R * CH / 128;          // 64-slot units per wave and phase
    constexpr int BUF = 4 * R * CH;           // slots (uint4) per buffer
    constexpr int XS = AL_PH / 32;            // X operands per phase
    const uint16_t* dsrc[UW];
#pragma unroll
    for (int i = 0; i < UW; ++i) {
      const int sl = 64 * (w * UW + i) + lane, q = sl / (CH * R), n = (sl / CH) % R;
      const int c = (sl % CH) ^ ((n >> 1) % CH);
      dsrc[i] = ((q & 1) ? l1lo : l1hi) + int64_t(n) * D + (q >> 1) * DH + 8 * c;
    }
    v8bf xa[AL_NB][XS];
    v4f acc[NT];
#pragma unroll
    for (int g = 0; g < NT; ++g) acc[g] = v4f{0, 0, 0, 0};
    // Issue order: the prologue loads phases 0 .. NB - 2 (slices, then X, per
    // phase); phase Q issues the loads of phase Q + NB - 1. Vector memory
    // operations retire in issue order, so the wait at the start of phase P
    // may leave in flight exactly the operations issued after the X
    // operands of P.
    constexpr auto al_pending = [](int ph) {
      int after = 0;
      for (int j = ph + 1; j <= AL_NB - 2 && j < NPH; ++j) after += UW + XS;   // prologue
      for (int q = 0; q < ph; ++q)                                             // phases before
        if (q + AL_NB - 1 < NPH && q + AL_NB - 1 > ph) after += UW + XS;
      return after;
    };
#define HQ_AL_LOAD(P_)                                                                      \
  if constexpr ((P_) < NPH) {                                                               \
    _Pragma("unroll") for (int i = 0; i < UW; ++i)                                          \
      lds_dma16(dsrc[i] + (P_) * AL_PH, &lds[((P_) % AL_NB) * BUF + 64 * (w * UW + i)]);    \
    _Pragma("unroll") for (int st = 0; st < XS; ++st)                                       \
      xa[(P_) % AL_NB][st] = *reinterpret_cast<const v8bf*>(xp + (P_) * AL_PH + 32 * st);   \
    __builtin_amdgcn_sched_barrier(0);                                                      \
  }
#define HQ_AL_PHASE(P_)                                                                     \
  if constexpr ((P_) < NPH) {                                                               \
    /* vmcnt(al_pending(P_)) lgkmcnt(0) */                                                  \
    __builtin_amdgcn_s_waitcnt((al_pending(P_) & 0xF) | ((al_pending(P_) >> 4) << 14) |     \
                               0x70);                                                       \
    /* every wave's slices of P_ are in LDS and buffer (P_ - 1) % NB is read; a */            \
    /* bare barrier: __syncthreads' release fence would wait for the DMA of the */           \
    /* later phases too */                                                                   \
    asm volatile("" ::: "memory");                                                          \
    __builtin_amdgcn_s_barrier();                                                           \
    asm volatile("" ::: "memory");                                                          \
    HQ_AL_LOAD((P_) + AL_NB - 1)                                                            \
    const uint4* const bq = &lds[((P_) % AL_NB) * BUF];                                     \
    _Pragma("unroll") for (int st = 0; st < XS; ++st)                                       \
      _Pragma("unroll") for (int g = 0; g < NT; ++g) {                                      \
        const int n = g * 16 + nl, ci = n * CH + ((4 * st + (lane >> 4)) ^ ((n >> 1) % CH)); \
        v4i bh, bl;                                                                         \
        lds_read2_b128(&bq[(2 * kh) * R * CH + ci], &bq[(2 * kh + 1) * R * CH + ci], bh, bl); \
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[(P_) % AL_NB][st],              \
                                                         __builtin_bit_cast(v8bf, bh), acc[g], 0, 0, 0); \
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[(P_) % AL_NB][st],              \
                                                         __builtin_bit_cast(v8bf, bl), acc[g], 0, 0, 0); \
      }                                                                                     \
  }
    static_assert(NPH <= 24 && AL_NB == 4, "phase sequence below");
    HQ_AL_LOAD(0) HQ_AL_LOAD(1) HQ_AL_LOAD(2)
    HQ_AL_PHASE(0) HQ_AL_PHASE(1) HQ_AL_PHASE(2) HQ_AL_PHASE(3) HQ_AL_PHASE(4) HQ_AL_PHASE(5)
    HQ_AL_PHASE(6) HQ_AL_PHASE(7) HQ_AL_PHASE(8) HQ_AL_PHASE(9) HQ_AL_PHASE(10) HQ_AL_PHASE(11)
    HQ_AL_PHASE(12) HQ_AL_PHASE(13) HQ_AL_PHASE(14) HQ_AL_PHASE(15) HQ_AL_PHASE(16)
    HQ_AL_PHASE(17) HQ_AL_PHASE(18) HQ_AL_PHASE(19) HQ_AL_PHASE(20) HQ_AL_PHASE(21)
    HQ_AL_PHASE(22) HQ_AL_PHASE(23)
#undef HQ_AL_PHASE
#undef HQ_AL_LOAD
    // the halves: the second writes its products, the first adds them
    // (16x16 output layout: lane l, register j -> row 4 (l / 16) + j, rank l % 16)
    __syncthreads();
    float* const red = reinterpret_cast<float*>(lds);
    if (kh == 1) {
#pragma unroll
      for (int g = 0; g < NT; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) red[(rg * 16 + 4 * (lane >> 4) + j) * R + g * 16 + nl] = acc[g][j];
    }
    __syncthreads();
    if (kh == 0) {
#pragma unroll
      for (int g = 0; g < NT; ++g)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int64_t m = rbase + 4 * (lane >> 4) + j;
          if (m < a.rows)
            U[m * R + g * 16 + nl] = acc[g][j] + red[(rg * 16 + 4 * (lane >> 4) + j) * R + g * 16 + nl];
        }
    }
    return;
  }

  // row transform of rows 8 (blockIdx.x - npb) + w (the row kernel's body)
  const int t = lane;
  const int64_t row = int64_t(int(blockIdx.x) - npb) * 8 + w;
  const bool valid = row < a.rows;
  const int64_t r = valid ? row : a.rows - 1;
  const uint16_t* src = static_cast<const uint16_t*>(a.in) + r * D + t * 8;
  float4* const lpar = reinterpret_cast<float4*>(lds);
  float v[E];
  if constexpr (P > 0) {
    float4 pv[PV];
#pragma unroll
    for (int k = 0; k < PV; ++k) {
      const int i = k * 512 + tid < NV4 ? k * 512 + tid : NV4 - 1;
      pv[k] = reinterpret_cast<const float4*>(a.scale)[i];
    }
#pragma unroll
    for (int c = 0; c < C; ++c) load8(src + c * 8 * G, &v[c * 8]);
#pragma unroll
    for (int k = 0; k < PV; ++k) lpar[k * 512 + tid] = pv[k];
    __syncthreads();
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) load8(src + c * 8 * G, &v[c * 8]);
  }
  row_fast_body<G, C, NX, P, 0>(a, inv_sqrt_b, t, row, valid, v, lpar);
}

bool act_lr_applies(const RowArgs& a, const RowGeom& g, int r) {
  const int nx = a.log2b - 9;
  return a.in_bf16 && a.mode == ROW_ACT && !a.group && !a.chan_mean && g.G == 64 &&
         (g.C == 5 || g.C == 6) && (r == 16 || r == 32) && nx >= 0 && (1 << nx) <= g.C &&
         g.C % (1 << nx) == 0;
}

template <int C, int NX, int NT>
static void launch_al_p(const RowArgs& a, dim3 grid, float isb, const uint16_t* hi,
                        const uint16_t* lo, float* U, int npb, hipStream_t s) {
  if (a.scale)
    hipLaunchKernelGGL((act_lr_kernel<C, NX, 1, NT>), grid, dim3(512), 0, s, a, isb, hi, lo, U, npb);
  else
    hipLaunchKernelGGL((act_lr_kernel<C, NX, 0, NT>), grid, dim3(512), 0, s, a, isb, hi, lo, U, npb);
}

template <int NT>
static hipError_t launch_al_nt(const RowArgs& a, const RowGeom& g, dim3 grid, float isb,
                               const uint16_t* hi, const uint16_t* lo, float* U, int npb,
                               hipStream_t s) {
  const int nx = a.log2b - 9;
  if (g.C == 5 && nx == 0) launch_al_p<5, 0, NT>(a, grid, isb, hi, lo, U, npb, s);
  else if (g.C == 6 && nx == 0) launch_al_p<6, 0, NT>(a, grid, isb, hi, lo, U, npb, s);
  else if (g.C == 6 && nx == 1) launch_al_p<6, 1, NT>(a, grid, isb, hi, lo, U, npb, s);
  else return hipErrorNotSupported;
  return hipGetLastError();
}

hipError_t launch_act_lr(const RowArgs& a, const RowGeom& g, int r, const uint16_t* l1_hi,
                         const uint16_t* l1_lo, float* U, hipStream_t s) {
  if (!act_lr_applies(a, g, r)) return hipErrorNotSupported;
  if (a.rows <= 0) return hipSuccess;
  const int64_t npb = (a.rows + AL_ROWS - 1) / AL_ROWS;
  const dim3 grid{unsigned(npb + (a.rows + 7) / 8)};
  const float isb = 1.0f / sqrtf(float(1 << a.log2b));
  if (r == 16) return launch_al_nt<1>(a, g, grid, isb, l1_hi, l1_lo, U, int(npb), s);
  return launch_al_nt<2>(a, g, grid, isb, l1_hi, l1_lo, U, int(npb), s);
}

}  // namespace hq
