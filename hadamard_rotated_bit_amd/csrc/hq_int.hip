// Integer-only layers with integer requantisation ("Hadamard-Domain Model
// Quantization for Learned Image Coding", Sec. IV-B Eq. (13)-(22) and
// supplement Eq. (40)-(44)). A weight-only Hadamard (WH) layer transforms the
// weight along its output channels, W-bar = H_out W, b-bar = b H_out, and
// takes its int8 activation in the original basis; a double-Hadamard (DH)
// layer transforms it along its input channels, W-bar = W H_in, b-bar = b,
// and takes its activation in the H_in basis. The int32 product
// a = x w-bar^T + b_int goes onto the next layer's int8 grid with integers
// only, through one unnormalised transform of order m over the channels
// (WH: restoring the original basis; DH: the next layer's H_in basis; m = 1:
// none):
//
//   y = clamp(round(H~_m (M . a) / 2^n), -127, 127)
//
// with per-channel 16-bit multipliers M and one shared shift n (the Hadamard
// normalisation 1/sqrt(m) folded into M). With an activation between the
// layers (Table I, Eq. (20)-(22); supplement Eq. (45)-(49)) a second
// transform H~_p (the next layer's H_in) follows it: ReLU keeps the single
// multiplier-shift pair (y = clamp(round(H~_p relu(H~_m (M . a)) / 2^n))),
// SiLU and GELU run on their own int8 grid through a 255-entry table:
// z = clamp(round(H~_m (M_out . a) / 2^n_out)), u = LUT[z],
// y = clamp(round(H~_p (M_in u) / 2^n_in)).
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }

// W-bar = H_m W over blocks of m output channels: block (x, y) of the grid
// takes columns [32 x, 32 x + 32) of rows [m y, m y + m) into LDS, runs the
// log2(m) butterfly stages over the row index and writes the rows times
// 1/sqrt(m) as float32. Rows at or past `rows` read as zeros (a padded
// order: W-bar = H_m [W; 0], supplement Eq. (40) with T_out = P H_m).
template <typename TW>
__global__ __launch_bounds__(256) void wh_weight_kernel(const TW* __restrict__ w, int rows,
                                                        int d_in, int m, float inv_sqrt_m,
                                                        float* __restrict__ wbar) {
  constexpr int CW = 32, LD = CW + 1;
  __shared__ float tile[WH_MAX_BLOCK * LD];
  const int col0 = blockIdx.x * CW;
  const int64_t row0 = int64_t(blockIdx.y) * m;
  const int tc = threadIdx.x & (CW - 1), tr = threadIdx.x / CW;   // 8 row lanes
  const int col = col0 + tc;
  for (int r = tr; r < m; r += 8)
    tile[r * LD + tc] =
        (col < d_in && row0 + r < rows) ? to_f32(w[(row0 + r) * d_in + col]) : 0.0f;
  __syncthreads();
  for (int h = 1; h < m; h <<= 1) {
    // m / 2 butterflies per column, (i, i + h) with bit h of i clear
    for (int p = tr; p < m / 2; p += 8) {
      const int i = (p / h) * 2 * h + (p % h);
      const float a = tile[i * LD + tc], b = tile[(i + h) * LD + tc];
      tile[i * LD + tc] = a + b;
      tile[(i + h) * LD + tc] = a - b;
    }
    __syncthreads();
  }
  if (col < d_in)
    for (int r = tr; r < m; r += 8) wbar[(row0 + r) * d_in + col] = tile[r * LD + tc] * inv_sqrt_m;
}

// out [rows, width] f32 = [w 0]: each row's d_in weights, then zeros up to
// width (a padded input order: W-bar = [W 0] H_m, supplement Eq. (39)).
template <typename TW>
__global__ __launch_bounds__(256) void pad_rows_kernel(const TW* __restrict__ w, int64_t rows,
                                                       int d_in, int width,
                                                       float* __restrict__ out) {
  const int64_t n = rows * width;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / width;
    const int c = int(i - r * width);
    out[i] = c < d_in ? to_f32(w[r * d_in + c]) : 0.0f;
  }
}

// Multiplier bound for transforms whose orders multiply to `orders` (a power
// of two): |a + b_int| < 2^28, so M < 2^(24 - log2 orders) keeps every
// integer below 2^52 through the unnormalised transforms.
__device__ __forceinline__ double int_mult_bound(int orders) {
  const int lg = 31 - __clz(orders);
  const double b = ldexp(1.0, 24 - lg) - 1.0;
  return b < double(WH_MULT_MAX) ? b : double(WH_MULT_MAX);
}

// The largest shift n <= WH_SHIFT_MAX with round(2^n top) <= bound (0 when
// top is 0).
__device__ __forceinline__ int int_shift_for(double top, double bound) {
  int n = 0;
  if (top > 0.0)
    while (n < WH_SHIFT_MAX && rint(ldexp(top, n + 1)) <= bound) ++n;
  return n;
}

// The activations of the table (float64).
__device__ __forceinline__ double int_phi(int act, double x) {
  if (act == 2) return x / (1.0 + exp(-x));                 // SiLU
  return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));              // GELU, x Phi(x)
}

// Offline constants (one block, float64): b-bar = b H_bb (bb = m for WH, 1
// for DH), s_A = s_x s_w, b_int = round(b-bar / s_A) (saturated at +-2^27,
// see the requantisation kernel), rho, the shared shift n (largest n <= 48
// with every round(2^n rho) within the multiplier bound) and M = round(2^n
// rho). Identity / ReLU: rho = s_A / (sqrt(m post) s_y), bound for m post.
// SiLU / GELU: rho = s_A / (sqrt(m) s_z), bound for m; then the table over
// z = -127 .. 127 (lut[z + 127] = clamp(round(phi(s_z z) / s_u)), lut[255] =
// 0) and M_in = round(2^n_in s_u / (sqrt(post) s_y)). d_out counts the
// accumulator channels (a padded WH order: m of them), n_bias the bias
// entries (the bias reads as zero past them); rows past d_out get zeros.
__global__ __launch_bounds__(256) void int_constants_kernel(
    const float* __restrict__ bias, int n_bias, const float* __restrict__ s_w, int d_out,
    int d_out_pad, int m, int post, int act, int bb_order, double s_x, double s_y, double s_z,
    double s_u,
    int32_t* __restrict__ b_int, int32_t* __restrict__ mult, int32_t* __restrict__ shift,
    int8_t* __restrict__ lut, int32_t* __restrict__ mult_in, int32_t* __restrict__ shift_in) {
  __shared__ double red[256];
  const bool general = act >= 2;
  const double sqm = sqrt(double(general ? m : m * post));
  const double s_den = general ? s_z : s_y;
  double top = 0.0;
  for (int c = threadIdx.x; c < d_out; c += 256) {
    const double rho = s_x * double(s_w[c]) / (sqm * s_den);
    top = rho > top ? rho : top;
  }
  red[threadIdx.x] = top;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if (int(threadIdx.x) < s)
      red[threadIdx.x] = red[threadIdx.x + s] > red[threadIdx.x] ? red[threadIdx.x + s]
                                                                 : red[threadIdx.x];
    __syncthreads();
  }
  top = red[0];
  const int n = int_shift_for(top, int_mult_bound(general ? m : m * post));
  if (threadIdx.x == 0) {
    *shift = n;
    int32_t mi = 0, ni = 0;
    if (general) {
      const double rho_in = s_u / (sqrt(double(post)) * s_y);
      ni = int_shift_for(rho_in, double(WH_MULT_MAX));
      mi = int32_t(rint(ldexp(rho_in, ni)));
    }
    *mult_in = mi;
    *shift_in = ni;
  }
  {
    const int t = threadIdx.x;   // one table entry per thread
    double q = 0.0;
    if (general && t < 255) {
      q = rint(int_phi(act, s_z * double(t - 127)) / s_u);
      q = q > 127.0 ? 127.0 : (q < -127.0 ? -127.0 : q);
    }
    lut[t] = int8_t(int(q));
  }
  for (int c = threadIdx.x; c < d_out_pad; c += 256) {
    int32_t bi = 0, mc = 0;
    if (c < d_out) {
      const double s_a = s_x * double(s_w[c]);
      const double rho = s_a / (sqm * s_den);
      mc = int32_t(rint(ldexp(rho, n)));
      if (bias && s_a > 0.0) {
        const int base = (c / bb_order) * bb_order, ci = c - base;
        double bb = 0.0;
        for (int k = 0; k < bb_order && base + k < n_bias; ++k) {
          const double v = double(bias[base + k]);
          bb += (__popc(ci & k) & 1) ? -v : v;
        }
        double q = rint((bb / sqrt(double(bb_order))) / s_a);
        q = q > double(WH_BIAS_MAX) ? double(WH_BIAS_MAX) : q;
        q = q < -double(WH_BIAS_MAX) ? -double(WH_BIAS_MAX) : q;
        bi = int32_t(q);
      }
    }
    b_int[c] = bi;
    mult[c] = mc;
  }
}

// The requantisation carries its integers in float64 registers: with
// |a + b_int| < 2^28 (|a| <= 127^2 d_in <= 2^27, |b_int| <= 2^27) and M below
// the bound for the transforms' orders (2^(24 - log2(m post))), every
// intermediate is an integer below 2^52 in magnitude (after a table, |M_in u|
// <= 127 * 32767 and 256 terms), so float64 additions, products, the scaling
// by 2^-n and round-to-nearest-even are exact and give the integer results
// bit for bit, at a quarter of the instructions 64-bit integer arithmetic
// needs on the VALU.

// Value of x held by lane l ^ D of the same 16-lane row (D = 1, 2, 4, 8):
// DPP quad permutes for 1 and 2, a DPP row rotation by 8 (its direction does
// not matter), and for 4 the swizzle's xor mode.
template <int D>
__device__ __forceinline__ int lane_xor16(int x) {
  static_assert(D == 1 || D == 2 || D == 4 || D == 8, "lane distance");
  if constexpr (D == 1) return __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
  if constexpr (D == 2) return __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
  if constexpr (D == 8) return __builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false);
  return __builtin_amdgcn_ds_swizzle(x, 0x1F | (4 << 10));
}

template <int D>
__device__ __forceinline__ double lane_xor16_f64(double v) {
  const uint64_t b = __builtin_bit_cast(uint64_t, v);
  const int lo = lane_xor16<D>(int(uint32_t(b)));
  const int hi = lane_xor16<D>(int(uint32_t(b >> 32)));
  return __builtin_bit_cast(double, (uint64_t(uint32_t(hi)) << 32) | uint64_t(uint32_t(lo)));
}

// One butterfly stage over channel bit 4 + log2(D) (lane distance D): the
// lane with bit D clear keeps u + partner, the other partner - u.
template <int D>
__device__ __forceinline__ void int_xstage(double (&u)[16], int lane, int m) {
  if (16 * D >= m) return;
  const double g = (lane & D) ? -1.0 : 1.0;
#pragma unroll
  for (int k = 0; k < 16; ++k) u[k] = fma(u[k], g, lane_xor16_f64<D>(u[k]));
}

// Butterflies of one 16-lane group's 256-channel unit (channel bits 0-3 in
// the lane, bits 4-7 across the group), for blocks of m channels.
__device__ __forceinline__ void int_unit_transform(double (&u)[16], int lane, int m) {
#pragma unroll
  for (int h = 1; h < 16; h <<= 1) {
    if (h < m) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        if (!(k & h)) {
          const double x = u[k], z = u[k + h];
          u[k] = x + z;
          u[k + h] = x - z;
        }
      }
    }
  }
  int_xstage<1>(u, lane, m);
  int_xstage<2>(u, lane, m);
  int_xstage<4>(u, lane, m);
  int_xstage<8>(u, lane, m);
}

// round(u 2^-n) with ties to even, clamped to +-127, as 16 int8 codes.
__device__ __forceinline__ uint4 int_unit_codes(const double (&u)[16], double scale) {
  uint32_t w[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t packed = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const double v = fmin(fmax(rint(u[4 * q + k] * scale), -127.0), 127.0);
      packed |= (uint32_t(int(v)) & 0xFFu) << (8 * k);
    }
    w[q] = packed;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// The transition on one unit, u = M . (acc + b_int) on entry (channels c0 ..
// c0 + 15 of the lane): H~_m, the projection onto the first `keep` channels,
// the activation, H~_post (channels past `keep` are the zero padding of a
// padded post order), then the final rounding as 16 int8 codes. ACT 0:
// identity, 1: ReLU (both with the one shift), 2: the table (SiLU, GELU):
// z = clamp(round(v / 2^n_out)), u = M_in lut[z + 127], final shift n_in.
template <int ACT>
__device__ __forceinline__ uint4 int_unit_transition(double (&u)[16], int lane, int c0,
                                                     const IntTransition& tr) {
  const double s1 = ldexp(1.0, -*tr.shift);
  int_unit_transform(u, lane, tr.m);
  // a padded WH order keeps its first `keep` channels (the projection P)
#pragma unroll
  for (int k = 0; k < 16; ++k)
    if (c0 + k >= tr.keep) u[k] = 0.0;
  if constexpr (ACT == 1) {
#pragma unroll
    for (int k = 0; k < 16; ++k) u[k] = fmax(u[k], 0.0);
  } else if constexpr (ACT == 2) {
    const double m_in = double(*tr.mult_in);
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const double z = fmin(fmax(rint(u[k] * s1), -127.0), 127.0);
      u[k] = c0 + k < tr.keep ? double(tr.lut[int(z) + 127]) * m_in : 0.0;
    }
  }
  int_unit_transform(u, lane, tr.post);
  return int_unit_codes(u, ACT == 2 ? ldexp(1.0, -*tr.shift_in) : s1);
}

// Requantisation of int32 products acc [T, ldc] (acc_w channels, without
// bias) into y [T, ldy] (out_w channels). Each group of
// 16 lanes takes one (token, 256-channel chunk) unit, lane l of the group
// holding channels 16 l .. 16 l + 15 of the chunk. u = M (acc + b_int), the
// unnormalised Sylvester butterflies over blocks of m channels (channel bits
// 0-3 inside the lane, bits 4-7 across the group's lanes), then
// round(u / 2^n) with ties to even and clamping to +-127. Every lane of a
// group runs the butterflies (invalid channels hold 0; blocks never mix valid
// and invalid channels, m dividing d_out).
template <int ACT>
__global__ __launch_bounds__(256) void int_requant_kernel(
    const int32_t* __restrict__ acc, int64_t ldc, int64_t T, int acc_w, int out_w, int chunks,
    IntTransition tr, int8_t* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 15;
  const int64_t unit = int64_t(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const bool live = unit < T * chunks;
  const int64_t uu = live ? unit : T * chunks - 1;
  const int64_t row = uu / chunks;
  const int c0 = int(uu - row * chunks) * 256 + 16 * lane;
  double u[16];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int c = c0 + 4 * q;
    if (c < acc_w) {   // acc_w % 8 == 0: whole runs of 4 are in or out
      const int4 a = *reinterpret_cast<const int4*>(acc + row * ldc + c);
      const int4 b = *reinterpret_cast<const int4*>(tr.b_int + c);
      const int4 mm = *reinterpret_cast<const int4*>(tr.mult + c);
      u[4 * q + 0] = double(a.x + b.x) * double(mm.x);
      u[4 * q + 1] = double(a.y + b.y) * double(mm.y);
      u[4 * q + 2] = double(a.z + b.z) * double(mm.z);
      u[4 * q + 3] = double(a.w + b.w) * double(mm.w);
    } else {
      u[4 * q + 0] = u[4 * q + 1] = u[4 * q + 2] = u[4 * q + 3] = 0.0;
    }
  }
  const uint4 w = int_unit_transition<ACT>(u, lane, c0, tr);
  if (!live || c0 >= out_w) return;
  int8_t* dst = y + row * ldy + c0;
  if (c0 + 16 <= out_w) {
    *reinterpret_cast<uint4*>(dst) = w;
  } else {   // the last 8 channels of out_w
    *reinterpret_cast<uint2*>(dst) = make_uint2(w.x, w.y);
  }
}

// The whole integer layer in one kernel for d_out a multiple of 256: block
// (bx, by) takes tokens 32 bx .. 32 bx + 31 and channels 256 by .. + 255.
// Each of the 8 waves forms its 32 x 32 part of a = x w-bar^T with
// v_mfma_i32_32x32x32_i8 (operands straight from memory: 8 k-steps of both
// operands in flight per round trip), the exact int32 tile goes to LDS, and
// the block then requantises it unit by unit as above (32 units, one per 16
// lanes), so the products never leave the chip.
typedef int iv4 __attribute__((ext_vector_type(4)));
typedef int iv16 __attribute__((ext_vector_type(16)));
constexpr int IF_ROWS = 32;
constexpr int IF_PITCH = 256 + 4;   // int32 per LDS row (16-B aligned, rows 4 banks apart)
template <int ACT>
__global__ __launch_bounds__(512) void int_fused_kernel(
    const int8_t* __restrict__ x, int64_t T, int d_in, const int8_t* __restrict__ w, int d_out,
    IntTransition tr, int8_t* __restrict__ y) {
  __shared__ __attribute__((aligned(16))) int32_t tile[IF_ROWS * IF_PITCH];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t row0 = int64_t(blockIdx.x) * IF_ROWS;
  const int c_blk = int(blockIdx.y) * 256;
  int64_t xr = row0 + (lane & 31);
  if (xr >= T) xr = T - 1;
  // MFMA operands: lane l feeds row l % 32 and k-bytes 16 (l / 32) .. + 15 of
  // each 32-byte k-step
  const int kh = 16 * (lane >> 5);
  const int8_t* xa = x + xr * d_in + kh;
  const int8_t* wb = w + int64_t(c_blk + 32 * wv + (lane & 31)) * d_in + kh;
  iv16 acc = {0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0};
  for (int k0 = 0; k0 < d_in; k0 += 256) {
    iv4 a[8], b[8];
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      if (k0 + 32 * st < d_in) {
        a[st] = *reinterpret_cast<const iv4*>(xa + k0 + 32 * st);
        b[st] = *reinterpret_cast<const iv4*>(wb + k0 + 32 * st);
      }
    }
#pragma unroll
    for (int st = 0; st < 8; ++st)
      if (k0 + 32 * st < d_in) acc = __builtin_amdgcn_mfma_i32_32x32x32_i8(b[st], a[st], acc, 0, 0, 0);
  }
  // lane l, register r: token l % 32, channel (of the wave's 32-wide tile)
  // 8 (r / 4) + 4 (l / 32) + r % 4
  int32_t* trow = tile + (lane & 31) * IF_PITCH + 32 * wv + 4 * (lane >> 5);
#pragma unroll
  for (int q = 0; q < 4; ++q)
    *reinterpret_cast<iv4*>(trow + 8 * q) =
        iv4{acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]};
  __syncthreads();
  const int l16 = tid & 15, cl = 16 * l16;
  {
    const int r = tid >> 4;   // 32 units, one per 16 lanes
    double u[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int c = c_blk + cl + 4 * q;
      const int4 av = *reinterpret_cast<const int4*>(tile + r * IF_PITCH + cl + 4 * q);
      const int4 bv = *reinterpret_cast<const int4*>(tr.b_int + c);
      const int4 mv = *reinterpret_cast<const int4*>(tr.mult + c);
      u[4 * q + 0] = double(av.x + bv.x) * double(mv.x);
      u[4 * q + 1] = double(av.y + bv.y) * double(mv.y);
      u[4 * q + 2] = double(av.z + bv.z) * double(mv.z);
      u[4 * q + 3] = double(av.w + bv.w) * double(mv.w);
    }
    const uint4 codes = int_unit_transition<ACT>(u, l16, c_blk + cl, tr);
    if (row0 + r < T) *reinterpret_cast<uint4*>(y + (row0 + r) * d_out + c_blk + cl) = codes;
  }
}

hipError_t launch_wh_weight(const void* w, int w_bf16, int d_out, int acc_rows, int d_in, int m,
                            float* wbar, hipStream_t s) {
  if (m < 1 || m > WH_MAX_BLOCK || (m & (m - 1)) || acc_rows % m || acc_rows < d_out)
    return hipErrorInvalidValue;
  dim3 grid{unsigned((d_in + 31) / 32), unsigned(acc_rows / m)};
  const float ism = 1.0f / sqrtf(float(m));
  if (w_bf16)
    hipLaunchKernelGGL(wh_weight_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(w), d_out, d_in, m, ism, wbar);
  else
    hipLaunchKernelGGL(wh_weight_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(w), d_out, d_in, m, ism, wbar);
  return hipGetLastError();
}

hipError_t launch_pad_rows(const void* w, int w_bf16, int64_t rows, int d_in, int width,
                           float* out, hipStream_t s) {
  if (rows <= 0) return hipSuccess;
  if (width < d_in) return hipErrorInvalidValue;
  const int64_t n = rows * width;
  const unsigned blocks = unsigned(n / 256 + 1 < 4096 ? n / 256 + 1 : 4096);
  if (w_bf16)
    hipLaunchKernelGGL(pad_rows_kernel<uint16_t>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const uint16_t*>(w), rows, d_in, width, out);
  else
    hipLaunchKernelGGL(pad_rows_kernel<float>, dim3(blocks), dim3(256), 0, s,
                       static_cast<const float*>(w), rows, d_in, width, out);
  return hipGetLastError();
}

hipError_t launch_int_constants(const float* bias, int n_bias, const float* s_w, int acc_w,
                                int d_out_pad, int m, int post, int act, int bias_block,
                                float s_x, float s_y, float s_z, float s_u, int32_t* b_int,
                                int32_t* mult, int32_t* shift, int8_t* lut, int32_t* mult_in,
                                int32_t* shift_in, hipStream_t s) {
  if (bias_block < 1 || (bias_block & (bias_block - 1)) || acc_w % bias_block || act < 0 ||
      act > 3 || post < 1 || (post & (post - 1)) || post > WH_MAX_BLOCK || n_bias > acc_w)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(int_constants_kernel, dim3(1), dim3(256), 0, s, bias, n_bias, s_w, acc_w,
                     d_out_pad, m, post, act, bias_block, double(s_x), double(s_y), double(s_z),
                     double(s_u), b_int, mult, shift, lut, mult_in, shift_in);
  return hipGetLastError();
}

// acc_w accumulator channels (whole blocks of m), keep <= acc_w of them
// after the projection, out_w output channels (whole blocks of post, at least
// keep); every width a multiple of 8.
static bool transition_ok(const IntTransition& tr, int acc_w, int out_w) {
  auto pow2 = [](int v) { return v >= 1 && v <= WH_MAX_BLOCK && !(v & (v - 1)); };
  return pow2(tr.m) && pow2(tr.post) && acc_w % tr.m == 0 && out_w % tr.post == 0 &&
         tr.keep >= 1 && tr.keep <= acc_w && tr.keep <= out_w && acc_w % 8 == 0 &&
         out_w % 8 == 0 && tr.act >= 0 && tr.act <= 3;
}

hipError_t launch_int_fused(const int8_t* x, int64_t T, int d_in, const int8_t* w, int d_out,
                            const IntTransition& tr, int8_t* y, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (d_out % 256 || d_in % 32 || tr.keep != d_out || !transition_ok(tr, d_out, d_out))
    return hipErrorInvalidValue;
  const dim3 grid{unsigned((T + IF_ROWS - 1) / IF_ROWS), unsigned(d_out / 256)};
  if (tr.act == 0)
    hipLaunchKernelGGL(int_fused_kernel<0>, grid, dim3(512), 0, s, x, T, d_in, w, d_out, tr, y);
  else if (tr.act == 1)
    hipLaunchKernelGGL(int_fused_kernel<1>, grid, dim3(512), 0, s, x, T, d_in, w, d_out, tr, y);
  else
    hipLaunchKernelGGL(int_fused_kernel<2>, grid, dim3(512), 0, s, x, T, d_in, w, d_out, tr, y);
  return hipGetLastError();
}

hipError_t launch_int_requant(const int32_t* acc, int64_t ldc, int64_t T, int acc_w, int out_w,
                              const IntTransition& tr, int8_t* y, int64_t ldy, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (!transition_ok(tr, acc_w, out_w) || ldc < acc_w || ldy < out_w) return hipErrorInvalidValue;
  const int chunks = ((acc_w > out_w ? acc_w : out_w) + 255) / 256;
  const int64_t units = T * chunks;   // 16 lanes each, 16 per block
  const dim3 grid{unsigned((units + 15) / 16)};
  if (tr.act == 0)
    hipLaunchKernelGGL(int_requant_kernel<0>, grid, dim3(256), 0, s, acc, ldc, T, acc_w, out_w,
                       chunks, tr, y, ldy);
  else if (tr.act == 1)
    hipLaunchKernelGGL(int_requant_kernel<1>, grid, dim3(256), 0, s, acc, ldc, T, acc_w, out_w,
                       chunks, tr, y, ldy);
  else
    hipLaunchKernelGGL(int_requant_kernel<2>, grid, dim3(256), 0, s, acc, ldc, T, acc_w, out_w,
                       chunks, tr, y, ldy);
  return hipGetLastError();
}

}  // namespace hq
