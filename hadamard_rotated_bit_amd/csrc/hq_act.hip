// Activation-side and offline kernels of libhq for gfx950:
//  * the fused per-row transform (scale -> fast Walsh-Hadamard transform ->
//    mean -> absmax -> symmetric quantise), used online for activations and
//    offline for the weights;
//  * per-channel absmax and the smoothing scale of HadaNorm Eq. (3);
//  * the low-rank down projection U = x' L1 (bf16 MFMA, split operands);
//  * small preparation helpers (fills, reciprocal, factor splitting).
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {

// ---------------------------------------------------------------------------
// Row geometry. A row of d channels is spread over G consecutive lanes of a
// wave; lane t holds C chunks of 8 consecutive channels:
//     channel e = c * 8G + t * 8 + j,   j in [0, 8), c in [0, C).
// Each chunk load is one coalesced 8G-channel segment per row. The bits of e
// split into j (3 bits, in registers), t (log2 G bits, across lanes) and c
// (in registers), so a butterfly stage of the Walsh-Hadamard transform on
// bit b is either an in-register add/sub pair or one cross-lane exchange.
// The smallest G that keeps C <= 8 (else C <= 16) is chosen: few cross-lane
// stages without giving up occupancy.
// ---------------------------------------------------------------------------
bool row_geometry(int d, RowGeom* g) {
  const int cands[3] = {16, 32, 64};
  for (int cap : {8, 16}) {          // prefer <= 64 values per lane (occupancy)
    for (int i = 0; i < 3; ++i) {
      const int G = cands[i];
      if (d % (8 * G)) continue;
      const int C = d / (8 * G);
      if (C >= 1 && C <= cap) {
        g->G = G;
        g->C = C;
        return true;
      }
    }
  }
  return false;
}

// Writes the lane's C chunks of codes (chunk c = channels c 8G + 8t .. +7) in
// the launch's code format: int8 bytes at row * d + channel, or E2M3 pieces
// in the row-group layout.
template <int G, int C>
__device__ __forceinline__ void store_codes(const RowArgs& a, int64_t row, int64_t base, int t,
                                            const float* v, float rcp) {
  if (a.code_fmt == CODES_E2M3) {
#pragma unroll
    for (int c = 0; c < C; ++c) store_e2m3x8<F6_GROUP>(a.codes, row, a.d, c * 8 * G + t * 8, &v[c * 8], rcp);
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float* vc = &v[c * 8];
      *reinterpret_cast<uint2*>(a.codes + base + c * 8 * G) =
          make_uint2(pack_codes4(vc[0], vc[1], vc[2], vc[3], rcp),
                     pack_codes4(vc[4], vc[5], vc[6], vc[7], rcp));
    }
  }
}

// One wave processes 64/G rows at once; a 256-thread block covers 4 waves.
//
// Per row (HadaNorm Eq. (1) activation side, HaTQ Eq. (3) quantiser):
//   x' = x * scale                      (scale = 1/sigma; sigma for weights)
//   y' = H~ x' per block                (unnormalised Sylvester butterflies;
//                                        1/sqrt(B) is folded into the scales)
//   mu' = sum(y') / d                   (if centring)
//   amax' = max |y' - mu'|
//   q = rint((y' - mu') * (qmax / amax'))  (fp32 operands, the exact product
//                                           rounded once, ties to even)
//   s = amax' / (sqrt(B) qmax),  mu = mu' / sqrt(B),  c = sum(y') / sqrt(B)
// Group-wise variant of store_codes (a.group = 64): chunk c of lane t lies in
// channel group c G/8 + t/8, shared by the 8 lanes t & ~7; each group is
// quantised with its own max |v| (a group maximum over those 8 lanes) and its
// scale written by the group's first lane to out_s[g * s_ld + row]. Every
// lane of the wave runs the cross-lane maxima; only valid rows store.
template <int G, int C>
__device__ __forceinline__ void store_group_codes(const RowArgs& a, int64_t row, int64_t base,
                                                  int t, const float* v, bool valid,
                                                  float inv_sqrt_b) {
  static_assert(G % 8 == 0, "8 lanes per 64-channel group");
  float rc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[c * 8 + j]));
    m = group_max<8>(m);
    rc[c] = m > 0.0f ? a.qmax / m : 0.0f;
    if (valid && (t & 7) == 0)
      a.out_s[int64_t(c * (G / 8) + t / 8) * a.s_ld + row] = m * inv_sqrt_b / a.qmax;
  }
  if (!valid) return;
  if (a.code_fmt == CODES_E2M3) {
#pragma unroll
    for (int c = 0; c < C; ++c) store_e2m3x8<F6_GROUP>(a.codes, row, a.d, c * 8 * G + t * 8, &v[c * 8], rc[c]);
  } else {
#pragma unroll
    for (int c = 0; c < C; ++c) {
      const float* vc = &v[c * 8];
      *reinterpret_cast<uint2*>(a.codes + base + c * 8 * G) =
          make_uint2(pack_codes4(vc[0], vc[1], vc[2], vc[3], rc[c]),
                     pack_codes4(vc[4], vc[5], vc[6], vc[7], rc[c]));
    }
  }
}

template <typename TIn, int G, int C>
__global__ __launch_bounds__(256) void row_transform_kernel(RowArgs a, float inv_sqrt_b) {
  constexpr int LOG2G = (G == 16) ? 4 : (G == 32) ? 5 : 6;
  constexpr int E = 8 * C;
  constexpr int RPW = 64 / G;
  const int lane = threadIdx.x & 63;
  const int t = lane & (G - 1);
  const int64_t row = (int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6)) * RPW + lane / G;
  const bool valid = row < a.rows;
  const int64_t r = valid ? row : a.rows - 1;
  const int d = a.d;
  const TIn* src = static_cast<const TIn*>(a.in) + r * d + t * 8;

  // Per-channel multiplier and mean first: loads retire in issue order, so
  // issuing them after the row would make the first chunk wait for all of it.
  float sc[E], sh[E];
  if (a.scale) {
#pragma unroll
    for (int c = 0; c < C; ++c) load8(a.scale + c * 8 * G + t * 8, &sc[c * 8]);
  }
  if (a.chan_mean) {
#pragma unroll
    for (int c = 0; c < C; ++c) load8(a.chan_mean + c * 8 * G + t * 8, &sh[c * 8]);
  }
  float v[E];
#pragma unroll
  for (int c = 0; c < C; ++c) load8(src + c * 8 * G, &v[c * 8]);

  // Chunk by chunk (so work on chunk c can start as soon as its load lands):
  // per-channel centring and scaling, then the butterflies on channel bits 0..2
  // (in registers) and 3 .. 3+log2G-1 (across lanes, on the VALU; the lower
  // partner keeps x+y, the upper x-y).
#pragma unroll
  for (int c = 0; c < C; ++c) {
    float* vc = &v[c * 8];
    if (a.chan_mean) {
#pragma unroll
      for (int j = 0; j < 8; ++j) vc[j] -= sh[c * 8 + j];
    }
    if (a.scale) {
#pragma unroll
      for (int j = 0; j < 8; ++j) vc[j] *= sc[c * 8 + j];
    }
#pragma unroll
    for (int b = 0; b < 3; ++b) {
      if (b < a.log2b) {
        const int h = 1 << b;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (!(e & h)) {
            const float x = vc[e], y = vc[e + h];
            vc[e] = x + y;
            vc[e + h] = x - y;
          }
        }
      }
    }
#define HQ_XSTAGE(BIT, M)                                                          \
    if (BIT < LOG2G && BIT + 3 < a.log2b) {                                        \
      const float sg = (t & M) ? -1.0f : 1.0f;                                     \
      _Pragma("unroll") for (int e = 0; e < 8; ++e) vc[e] = butterfly<M>(vc[e], sg); \
    }
    HQ_XSTAGE(0, 1)
    HQ_XSTAGE(1, 2)
    HQ_XSTAGE(2, 4)
    HQ_XSTAGE(3, 8)
    if constexpr (G >= 32) { HQ_XSTAGE(4, 16) }
    if constexpr (G >= 64) { HQ_XSTAGE(5, 32) }
#undef HQ_XSTAGE
  }
  // Remaining bits index chunks (in registers).
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int h = 1 << b;
    if (h < C && b + 3 + LOG2G < a.log2b) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        if (!(c & h) && c + h < C) {
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const float x = v[c * 8 + j], y = v[(c + h) * 8 + j];
            v[c * 8 + j] = x + y;
            v[(c + h) * 8 + j] = x - y;
          }
        }
      }
    }
  }

  // Row sum (bit-identical on every lane of the row).
  float sum = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) sum += v[e];
  sum = group_sum<G>(sum);

  const int64_t base = row * d + t * 8;
  if (a.mode == ROW_WEIGHT && a.group) {
    store_group_codes<G, C>(a, row, base, t, v, valid, inv_sqrt_b);
    if (valid && t == 0 && a.out_aux) a.out_aux[row] = sum * inv_sqrt_b;
    return;
  }
  if (a.mode == ROW_WEIGHT) {
    float amax = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) amax = fmaxf(amax, fabsf(v[e]));
    amax = group_max<G>(amax);
    const float rcp = amax > 0.0f ? a.qmax / amax : 0.0f;
    if (valid) {
      store_codes<G, C>(a, row, base, t, v, rcp);
      if (t == 0) {
        a.out_s[row] = amax * inv_sqrt_b / a.qmax;
        if (a.out_aux) a.out_aux[row] = sum * inv_sqrt_b;
      }
    }
    return;
  }

  // Centre in place; the absmax of the centred row follows.
  const float mu = a.center ? sum / float(d) : 0.0f;
  float amax = 0.0f;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    v[e] -= mu;
    amax = fmaxf(amax, fabsf(v[e]));
  }
  if (a.mode == ROW_EXPORT) {
    if (valid) {
#pragma unroll
      for (int c = 0; c < C; ++c) {
        float* o = a.out_xt + base + c * 8 * G;
        reinterpret_cast<float4*>(o)[0] =
            make_float4(v[c * 8 + 0] * inv_sqrt_b, v[c * 8 + 1] * inv_sqrt_b,
                        v[c * 8 + 2] * inv_sqrt_b, v[c * 8 + 3] * inv_sqrt_b);
        reinterpret_cast<float4*>(o)[1] =
            make_float4(v[c * 8 + 4] * inv_sqrt_b, v[c * 8 + 5] * inv_sqrt_b,
                        v[c * 8 + 6] * inv_sqrt_b, v[c * 8 + 7] * inv_sqrt_b);
      }
      if (t == 0 && a.out_aux) a.out_aux[row] = mu * inv_sqrt_b;
    }
    return;
  }

  if (a.group) {
    store_group_codes<G, C>(a, row, base, t, v, valid, inv_sqrt_b);
    if (valid && t == 0 && a.out_aux) a.out_aux[row] = mu * inv_sqrt_b;
    return;
  }
  amax = group_max<G>(amax);
  const float rcp = amax > 0.0f ? a.qmax / amax : 0.0f;
  if (valid) {
    store_codes<G, C>(a, row, base, t, v, rcp);
    if (t == 0) {
      a.out_s[row] = amax * inv_sqrt_b / a.qmax;
      if (a.out_aux) a.out_aux[row] = mu * inv_sqrt_b;
    }
  }
}

template <typename TIn, int G>
static hipError_t launch_row_g(const RowArgs& a, int C, hipStream_t s) {
  const int rpw = 64 / G;
  const int64_t blocks = (a.rows + 4 * rpw - 1) / (4 * rpw);
  const float isb = 1.0f / sqrtf(float(1 << a.log2b));
  dim3 grid{unsigned(blocks)}, block{256};
#define HQ_ROW_CASE(CC)                                                        \
  case CC:                                                                     \
    hipLaunchKernelGGL((row_transform_kernel<TIn, G, CC>), grid, block, 0, s, a, isb); \
    break;
  switch (C) {
    HQ_ROW_CASE(1) HQ_ROW_CASE(2) HQ_ROW_CASE(3) HQ_ROW_CASE(4)
    HQ_ROW_CASE(5) HQ_ROW_CASE(6) HQ_ROW_CASE(7) HQ_ROW_CASE(8)
    HQ_ROW_CASE(9) HQ_ROW_CASE(10) HQ_ROW_CASE(11) HQ_ROW_CASE(12)
    HQ_ROW_CASE(13) HQ_ROW_CASE(14) HQ_ROW_CASE(15) HQ_ROW_CASE(16)
    default:
      return hipErrorInvalidValue;
  }
#undef HQ_ROW_CASE
  return hipGetLastError();
}

hipError_t launch_row_transform(const RowArgs& a, hipStream_t s) {
  RowGeom g;
  if (!row_geometry(a.d, &g)) return hipErrorInvalidValue;
  if (a.rows <= 0) return hipSuccess;
  const hipError_t fe = launch_row_fast(a, g, s);
  if (fe != hipErrorNotSupported) return fe;
  if (a.in_bf16) {
    if (g.G == 16) return launch_row_g<uint16_t, 16>(a, g.C, s);
    if (g.G == 32) return launch_row_g<uint16_t, 32>(a, g.C, s);
    return launch_row_g<uint16_t, 64>(a, g.C, s);
  }
  if (g.G == 16) return launch_row_g<float, 16>(a, g.C, s);
  if (g.G == 32) return launch_row_g<float, 32>(a, g.C, s);
  return launch_row_g<float, 64>(a, g.C, s);
}

// ---------------------------------------------------------------------------
// Per-channel absmax over rows (calibration statistic of HadaNorm Eq. (3)).
// Thread = 8 consecutive channels over a strip of rows; strips combine with an
// unsigned atomic max on the float bit patterns (valid for values >= 0).
// ---------------------------------------------------------------------------
template <typename TIn>
__global__ __launch_bounds__(256) void col_absmax_kernel(const TIn* __restrict__ in, int64_t rows,
                                                         int d, int64_t strip,
                                                         uint32_t* __restrict__ out) {
  const int g = blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= d / 8) return;
  const int64_t r0 = int64_t(blockIdx.y) * strip;
  const int64_t r1 = r0 + strip < rows ? r0 + strip : rows;
  float m[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int64_t r = r0; r < r1; ++r) {
    float v[8];
    load8(in + r * d + g * 8, v);
#pragma unroll
    for (int j = 0; j < 8; ++j) m[j] = fmaxf(m[j], fabsf(v[j]));
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) atomicMax(out + g * 8 + j, __float_as_uint(m[j]));
}

hipError_t launch_col_absmax(const void* in, int in_bf16, int64_t rows, int d, float* absmax,
                             hipStream_t s) {
  hipError_t e = launch_fill_u32(reinterpret_cast<uint32_t*>(absmax), 0u, size_t(d), s);
  if (e != hipSuccess || rows <= 0) return e;
  const int64_t strip = 64;
  const int64_t strips = (rows + strip - 1) / strip;
  dim3 grid{unsigned((d / 8 + 255) / 256), unsigned(strips)}, block{256};
  if (in_bf16)
    hipLaunchKernelGGL(col_absmax_kernel<uint16_t>, grid, block, 0, s,
                       static_cast<const uint16_t*>(in), rows, d, strip,
                       reinterpret_cast<uint32_t*>(absmax));
  else
    hipLaunchKernelGGL(col_absmax_kernel<float>, grid, block, 0, s, static_cast<const float*>(in),
                       rows, d, strip, reinterpret_cast<uint32_t*>(absmax));
  return hipGetLastError();
}

__global__ void sigma_finish_kernel(const float* __restrict__ ax, float alpha, float eps, int d,
                                    float* __restrict__ sigma) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= d) return;
  const float aw = sigma[i];
  sigma[i] = powf(fmaxf(ax[i], eps), alpha) / powf(fmaxf(aw, eps), 1.0f - alpha);
}

hipError_t launch_sigma_finish(const float* ax, float alpha, float eps, int d, float* sigma,
                               hipStream_t s) {
  hipLaunchKernelGGL(sigma_finish_kernel, dim3((d + 255) / 256), dim3(256), 0, s, ax, alpha, eps, d,
                     sigma);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small helpers (kernels rather than hipMemset/hipMemcpy so that a caller may
// capture them in a graph).
// ---------------------------------------------------------------------------
__global__ void fill_u32_kernel(uint32_t* p, uint32_t v, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = v;
}
__global__ void fill_u8_kernel(uint8_t* p, uint8_t v, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += size_t(gridDim.x) * blockDim.x)
    p[i] = v;
}
__global__ void copy_f32_kernel(const float* src, float* dst, size_t n) {
  for (size_t i = size_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n;
       i += size_t(gridDim.x) * blockDim.x)
    dst[i] = src[i];
}
__global__ void reciprocal_kernel(const float* src, float* dst, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = 1.0f / src[i];
}

static unsigned grid_for(size_t n) {
  size_t b = (n + 255) / 256;
  if (b > 4096) b = 4096;
  return unsigned(b ? b : 1);
}

hipError_t launch_fill_u32(uint32_t* p, uint32_t v, size_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(fill_u32_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}
hipError_t launch_fill_u8(uint8_t* p, uint8_t v, size_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(fill_u8_kernel, dim3(grid_for(n)), dim3(256), 0, s, p, v, n);
  return hipGetLastError();
}
hipError_t launch_copy_f32(const float* src, float* dst, size_t n, hipStream_t s) {
  if (!n) return hipSuccess;
  hipLaunchKernelGGL(copy_f32_kernel, dim3(grid_for(n)), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}
hipError_t launch_reciprocal(const float* src, float* dst, int n, hipStream_t s) {
  hipLaunchKernelGGL(reciprocal_kernel, dim3((n + 255) / 256), dim3(256), 0, s, src, dst, n);
  return hipGetLastError();
}

struct Header256 {
  uint32_t w[64];
};
__global__ void write_header_kernel(Header256 h, uint32_t* dst) {
  if (threadIdx.x < 64) dst[threadIdx.x] = h.w[threadIdx.x];
}
hipError_t launch_write_header(const void* host_hdr, size_t bytes, void* dst, hipStream_t s) {
  if (bytes > sizeof(Header256)) return hipErrorInvalidValue;
  Header256 h = {};
  const uint8_t* src = static_cast<const uint8_t*>(host_hdr);
  uint8_t* hb = reinterpret_cast<uint8_t*>(h.w);
  for (size_t i = 0; i < bytes; ++i) hb[i] = src[i];
  hipLaunchKernelGGL(write_header_kernel, dim3(1), dim3(64), 0, s, h, static_cast<uint32_t*>(dst));
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Low-rank factor preparation: split fp32 values into bf16 hi + bf16 lo so a
// bf16 MFMA product keeps ~16 significant bits.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void split_bf16(float v, uint16_t* hi, uint16_t* lo) {
  const uint16_t h = f32_to_bf16(v);
  *hi = h;
  *lo = f32_to_bf16(v - bf16_to_f32(h));
}

template <typename TIn>
__device__ __forceinline__ float load1(const TIn* p, int64_t i);
template <>
__device__ __forceinline__ float load1<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p, int64_t i) {
  return bf16_to_f32(p[i]);
}

// out[k, i] = l1[i, k] / sigma_i  (transposed to K-contiguous rows)
template <typename TIn>
__global__ void prep_l1_kernel(const TIn* __restrict__ l1, const float* __restrict__ sinv, int d,
                               int r, uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(d) * r) return;
  const int k = int(idx / d), i = int(idx % d);
  const float v = load1(l1, int64_t(i) * r + k) * (sinv ? sinv[i] : 1.0f);
  split_bf16(v, hi + idx, lo + idx);
}
// out[j, k] = l2[k, j] for j < n; zero rows up to n_pad
template <typename TIn>
__global__ void prep_l2_kernel(const TIn* __restrict__ l2, int r, int n, int n_pad,
                               uint16_t* __restrict__ hi, uint16_t* __restrict__ lo) {
  const int64_t idx = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= int64_t(n_pad) * r) return;
  const int j = int(idx / r), k = int(idx % r);
  const float v = j < n ? load1(l2, int64_t(k) * n + j) : 0.0f;
  split_bf16(v, hi + idx, lo + idx);
}

hipError_t launch_prep_l1(const void* l1, int bf16, const float* sigma_inv, int d, int r,
                          uint16_t* hi, uint16_t* lo, hipStream_t s) {
  const int64_t n = int64_t(d) * r;
  dim3 grid{unsigned((n + 255) / 256)}, block{256};
  if (bf16)
    hipLaunchKernelGGL(prep_l1_kernel<uint16_t>, grid, block, 0, s,
                       static_cast<const uint16_t*>(l1), sigma_inv, d, r, hi, lo);
  else
    hipLaunchKernelGGL(prep_l1_kernel<float>, grid, block, 0, s, static_cast<const float*>(l1),
                       sigma_inv, d, r, hi, lo);
  return hipGetLastError();
}
hipError_t launch_prep_l2(const void* l2, int bf16, int r, int n, int n_pad, uint16_t* hi,
                          uint16_t* lo, hipStream_t s) {
  const int64_t tot = int64_t(n_pad) * r;
  dim3 grid{unsigned((tot + 255) / 256)}, block{256};
  if (bf16)
    hipLaunchKernelGGL(prep_l2_kernel<uint16_t>, grid, block, 0, s,
                       static_cast<const uint16_t*>(l2), r, n, n_pad, hi, lo);
  else
    hipLaunchKernelGGL(prep_l2_kernel<float>, grid, block, 0, s, static_cast<const float*>(l2), r,
                       n, n_pad, hi, lo);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Low-rank down projection U = x . (l1_hi + l1_lo)^T  (blog steps 3-4: the
// 16-bit branch sees the smoothed, un-rotated input; 1/sigma is folded into
// l1). v_mfma_f32_16x16x32_bf16: lane l supplies row (l % 16), channels
// 8*(l/16) .. +8 of a 32-channel step; B likewise with the rank index.
// A block of W waves owns 16 rows; the waves split the channels into W
// contiguous parts and add their partial 16 x R tiles through LDS. Each wave
// loads the operands of U steps before their products, so U memory round
// trips overlap instead of one per step.
// fp32 inputs are split into bf16 hi + lo as well (3 products).
// ---------------------------------------------------------------------------
template <typename TIn, int R>
__device__ __forceinline__ void lowrank_load_a(const TIn* __restrict__ x, int64_t off, v8bf* hi,
                                               v8bf* lo) {
  if constexpr (sizeof(TIn) == 2) {
    *hi = *reinterpret_cast<const v8bf*>(x + off);
  } else {
    float f[8];
    load8(reinterpret_cast<const float*>(x) + off, f);
    uint16_t h[8], l[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) split_bf16(f[j], &h[j], &l[j]);
    *hi = *reinterpret_cast<v8bf*>(h);
    *lo = *reinterpret_cast<v8bf*>(l);
  }
}

template <typename TIn, int R, int W>
__global__ __launch_bounds__(W * 64) void lowrank_down_kernel(const TIn* __restrict__ x,
                                                              int64_t rows, int d,
                                                              const uint16_t* __restrict__ l1hi,
                                                              const uint16_t* __restrict__ l1lo,
                                                              float* __restrict__ U) {
  constexpr int NG = R / 16, UN = 4;
  __shared__ float red[W][16][R + 1];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int64_t row0 = int64_t(blockIdx.x) * 16;
  int64_t row = row0 + (lane & 15);
  if (row >= rows) row = rows - 1;
  const int kq = (lane >> 4) * 8;
  v4f acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = v4f{0, 0, 0, 0};
  const int kbeg = w * (d / W), kend = kbeg + d / W;
  auto step = [&](const v8bf& ahi, const v8bf& alo, const v8bf (&bhi)[NG], const v8bf (&blo)[NG]) {
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, bhi[g], acc[g], 0, 0, 0);
      acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi, blo[g], acc[g], 0, 0, 0);
      if constexpr (sizeof(TIn) == 4)
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo, bhi[g], acc[g], 0, 0, 0);
    }
  };
  int k0 = kbeg;
  for (; k0 + 32 * UN <= kend; k0 += 32 * UN) {
    v8bf ahi[UN], alo[UN], bhi[UN][NG], blo[UN][NG];
#pragma unroll
    for (int u = 0; u < UN; ++u) {
      lowrank_load_a<TIn, R>(x, row * d + k0 + 32 * u + kq, &ahi[u], &alo[u]);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int64_t off = int64_t(g * 16 + (lane & 15)) * d + k0 + 32 * u + kq;
        bhi[u][g] = *reinterpret_cast<const v8bf*>(l1hi + off);
        blo[u][g] = *reinterpret_cast<const v8bf*>(l1lo + off);
      }
    }
    __builtin_amdgcn_sched_barrier(0);   // every load of the group issues before the products
#pragma unroll
    for (int u = 0; u < UN; ++u) step(ahi[u], alo[u], bhi[u], blo[u]);
  }
  for (; k0 < kend; k0 += 32) {
    v8bf ahi, alo, bhi[NG], blo[NG];
    lowrank_load_a<TIn, R>(x, row * d + k0 + kq, &ahi, &alo);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      const int64_t off = int64_t(g * 16 + (lane & 15)) * d + k0 + kq;
      bhi[g] = *reinterpret_cast<const v8bf*>(l1hi + off);
      blo[g] = *reinterpret_cast<const v8bf*>(l1lo + off);
    }
    step(ahi, alo, bhi, blo);
  }
  // 16x16 output layout: lane l, register i -> row 4*(l/16) + i, column l % 16.
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[w][4 * (lane >> 4) + i][g * 16 + (lane & 15)] = acc[g][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < 16 * R; idx += W * 64) {
    const int rr = idx / R, cc = idx % R;
    float sum = 0.0f;
#pragma unroll
    for (int q = 0; q < W; ++q) sum += red[q][rr][cc];
    if (row0 + rr < rows) U[(row0 + rr) * R + cc] = sum;
  }
}

// Split form of the down projection: block (bx, q) takes rows 128 bx ..
// 128 bx + 127 (16 per wave) over slice q of d (kw = d / KS channels). The
// block stages the slice of l1 (hi and lo, R rows) in LDS with a pitch of
// kw / 8 + 1 chunks of 16 B (the 16 rows one read phase touches land on 16
// distinct bank groups); every load of the block (the row's kw channels and
// the slice) issues before the first wait, so a wave makes one round trip.
// Each wave runs the one-pass kernel's MFMA sequence for its slice and
// writes its 16 x R products to part[q].
constexpr int LR_MAX_STEPS = 16;   // kw <= 512
constexpr int LR_FILL = 8;         // 16-B chunks of the slice per thread
template <typename TIn, int R>
__global__ __launch_bounds__(512) void lowrank_part_kernel(const TIn* __restrict__ x,
                                                           int64_t rows, int d, int kw,
                                                           const uint16_t* __restrict__ l1hi,
                                                           const uint16_t* __restrict__ l1lo,
                                                           float* __restrict__ part) {
  constexpr int NG = R / 16;
  extern __shared__ __attribute__((aligned(16))) uint4 lsl[];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int q = blockIdx.y, kbeg = q * kw, cpr = kw / 8, pitch = cpr + 1;
  const int nch = R * cpr;           // chunks per array
  // the slice: chunk i of array a (row i / cpr, chunk i % cpr), clamped
  // repeats past the end (same value to the same place)
  uint4 fv[LR_FILL];
  int fpos[LR_FILL];
#pragma unroll
  for (int j = 0; j < LR_FILL; ++j) {
    int i = j * 512 + tid;
    if (i > 2 * nch - 1) i = 2 * nch - 1;
    const int a = i >= nch ? 1 : 0, ii = i - a * nch, r = ii / cpr, c = ii - r * cpr;
    const uint16_t* src = (a ? l1lo : l1hi) + int64_t(r) * d + kbeg + 8 * c;
    fv[j] = *reinterpret_cast<const uint4*>(src);
    fpos[j] = a * R * pitch + r * pitch + c;
  }
  const int64_t row0 = int64_t(blockIdx.x) * 128 + 16 * w;
  int64_t row = row0 + (lane & 15);
  if (row >= rows) row = rows - 1;
  const int kq = (lane >> 4) * 8;
  const int steps = kw / 32;
  v8bf ahi[LR_MAX_STEPS], alo[LR_MAX_STEPS];
#pragma unroll
  for (int st = 0; st < LR_MAX_STEPS; ++st)
    if (st < steps) lowrank_load_a<TIn, R>(x, row * d + kbeg + 32 * st + kq, &ahi[st], &alo[st]);
#pragma unroll
  for (int j = 0; j < LR_FILL; ++j) lsl[fpos[j]] = fv[j];
  __syncthreads();
  v4f acc[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) acc[g] = v4f{0, 0, 0, 0};
#pragma unroll
  for (int st = 0; st < LR_MAX_STEPS; ++st) {
    if (st < steps) {
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        const int p = (g * 16 + (lane & 15)) * pitch + 4 * st + (lane >> 4);
        const v8bf bhi = *reinterpret_cast<const v8bf*>(&lsl[p]);
        const v8bf blo = *reinterpret_cast<const v8bf*>(&lsl[R * pitch + p]);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[st], bhi, acc[g], 0, 0, 0);
        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ahi[st], blo, acc[g], 0, 0, 0);
        if constexpr (sizeof(TIn) == 4)
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(alo[st], bhi, acc[g], 0, 0, 0);
      }
    }
  }
  // 16x16 output layout: lane l, register i -> row 4 (l / 16) + i, column l % 16.
  float* pq = part + int64_t(q) * rows * R;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t rr = row0 + 4 * (lane >> 4) + i;
    if (rr < rows) {
#pragma unroll
      for (int g = 0; g < NG; ++g) pq[rr * R + g * 16 + (lane & 15)] = acc[g][i];
    }
  }
}

// U = sum over the KS slices in order, from 0 (the one-pass kernel's
// order); the KS loads of an element issue together.
template <int KS>
__global__ void lowrank_sum_kernel(const float* __restrict__ part, int64_t n,
                                   float* __restrict__ U) {
  const int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i >= n) return;
  float p[KS];
#pragma unroll
  for (int q = 0; q < KS; ++q) p[q] = part[q * n + i];
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < KS; ++q) s += p[q];
  U[i] = s;
}

// Waves of the one-pass kernel where the split form does not apply.
static int lowrank_waves(int d) { return d % 256 == 0 && d >= 1024 ? 8 : 4; }

constexpr int LR_LDS_MAX = 81920;   // LDS of one split-form block (two fit on a CU)
constexpr int LR_CUS = 256;         // compute units the split form is balanced for

int lowrank_slices(int d, int r, int64_t rows) {
  if (d % 128 || (r != 16 && r != 32 && r != 48 && r != 64)) return 0;
  // Among 4, 6 and 8 slices of whole 32-channel steps that the block's
  // registers and LDS hold, the one with the least work per slice times
  // rounds of blocks over the compute units (ties: fewer slices).
  const int64_t row_blocks = (rows + 127) / 128;
  int best = 0;
  int64_t best_cost = 0;
  for (int ks : {4, 6, 8}) {
    const int kw = d / ks;
    if ((d / 32) % ks || kw / 32 > LR_MAX_STEPS || 2 * r * (kw / 8) > LR_FILL * 512 ||
        2 * r * (kw / 8 + 1) * 16 > LR_LDS_MAX)
      continue;
    const int64_t cost = (row_blocks * ks + LR_CUS - 1) / LR_CUS * kw;
    if (!best || cost < best_cost) {
      best = ks;
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_lowrank_split(const void* x, int x_bf16, int64_t rows, int d, int r,
                                const uint16_t* l1_hi, const uint16_t* l1_lo, float* part,
                                float* U, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  const int ks = lowrank_slices(d, r, rows);
  if (!ks) return hipErrorInvalidValue;
  const int kw = d / ks;
  const size_t lds = size_t(2) * r * (kw / 8 + 1) * 16;
  dim3 grid{unsigned((rows + 127) / 128), unsigned(ks)};
#define HQ_LRS(RR)                                                                              \
  case RR:                                                                                      \
    if (x_bf16)                                                                                 \
      hipLaunchKernelGGL((lowrank_part_kernel<uint16_t, RR>), grid, dim3(512), lds, s,          \
                         static_cast<const uint16_t*>(x), rows, d, kw, l1_hi, l1_lo, part);     \
    else                                                                                        \
      hipLaunchKernelGGL((lowrank_part_kernel<float, RR>), grid, dim3(512), lds, s,             \
                         static_cast<const float*>(x), rows, d, kw, l1_hi, l1_lo, part);        \
    break;
  switch (r) {
    HQ_LRS(16) HQ_LRS(32) HQ_LRS(48) HQ_LRS(64)
    default:
      return hipErrorInvalidValue;
  }
#undef HQ_LRS
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t n = rows * r;
  const dim3 sg{unsigned((n + 255) / 256)};
  if (ks == 8)
    hipLaunchKernelGGL(lowrank_sum_kernel<8>, sg, dim3(256), 0, s, part, n, U);
  else if (ks == 6)
    hipLaunchKernelGGL(lowrank_sum_kernel<6>, sg, dim3(256), 0, s, part, n, U);
  else
    hipLaunchKernelGGL(lowrank_sum_kernel<4>, sg, dim3(256), 0, s, part, n, U);
  return hipGetLastError();
}

hipError_t launch_lowrank_down(const void* x, int x_bf16, int64_t rows, int d, int r,
                               const uint16_t* l1_hi, const uint16_t* l1_lo, float* U,
                               hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (d % 128) return hipErrorInvalidValue;
  // one wave per slice of the split form (the same partition, so the same
  // bits), else eight waves per 16 rows when every wave still gets whole
  // 32-channel steps, else four
  const int ks = lowrank_slices(d, r, rows);
  const int waves = ks ? ks : lowrank_waves(d);
  dim3 grid{unsigned((rows + 15) / 16)};
#define HQ_LR_LAUNCH(RR, WW)                                                                    \
  if (x_bf16)                                                                                   \
    hipLaunchKernelGGL((lowrank_down_kernel<uint16_t, RR, WW>), grid, dim3(WW * 64), 0, s,       \
                       static_cast<const uint16_t*>(x), rows, d, l1_hi, l1_lo, U);              \
  else                                                                                          \
    hipLaunchKernelGGL((lowrank_down_kernel<float, RR, WW>), grid, dim3(WW * 64), 0, s,          \
                       static_cast<const float*>(x), rows, d, l1_hi, l1_lo, U);
#define HQ_LR_CASE(RR)                                                                          \
  case RR:                                                                                      \
    if (waves == 8) { HQ_LR_LAUNCH(RR, 8) }                                                    \
    else if (waves == 6) { HQ_LR_LAUNCH(RR, 6) }                                               \
    else { HQ_LR_LAUNCH(RR, 4) }                                                               \
    break;
  switch (r) {
    HQ_LR_CASE(16) HQ_LR_CASE(32) HQ_LR_CASE(48) HQ_LR_CASE(64)
    default:
      return hipErrorInvalidValue;
  }
#undef HQ_LR_CASE
#undef HQ_LR_LAUNCH
  return hipGetLastError();
}

}  // namespace hq
