// Weight-only Hadamard (WH) layer with integer requantisation ("Hadamard-Domain
// Model Quantization for Learned Image Coding", Sec. IV-B Eq. (15)-(22) and
// supplement Eq. (40)-(44)): the weight is transformed along its output
// channels, W-bar = H_out W, b-bar = b H_out; the int8 activation stays in its
// original basis; the int32 product a = x w-bar^T + b_int is mapped back to
// the original basis and onto the next layer's int8 grid with integers only:
//
//   y = clamp(round(H~_out (M . a) / 2^n), -127, 127)
//
// with per-channel 16-bit multipliers M and one shared shift n (the Hadamard
// normalisation 1/sqrt(m) folded into M).
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return bf16_to_f32(v); }

// W-bar = H_m W over blocks of m output channels: block (x, y) of the grid
// takes columns [32 x, 32 x + 32) of rows [m y, m y + m) into LDS, runs the
// log2(m) butterfly stages over the row index and writes the rows times
// 1/sqrt(m) as float32.
template <typename TW>
__global__ __launch_bounds__(256) void wh_weight_kernel(const TW* __restrict__ w, int d_in,
                                                        int m, float inv_sqrt_m,
                                                        float* __restrict__ wbar) {
  constexpr int CW = 32, LD = CW + 1;
  __shared__ float tile[WH_MAX_BLOCK * LD];
  const int col0 = blockIdx.x * CW;
  const int64_t row0 = int64_t(blockIdx.y) * m;
  const int tc = threadIdx.x & (CW - 1), tr = threadIdx.x / CW;   // 8 row lanes
  const int col = col0 + tc;
  for (int r = tr; r < m; r += 8)
    tile[r * LD + tc] = col < d_in ? to_f32(w[(row0 + r) * d_in + col]) : 0.0f;
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

// Offline constants (one block, float64): b-bar = b H_m, s_A = s_x s_w,
// b_int = round(b-bar / s_A) (saturated at +-2^30 so that a + b_int fits an
// int32), rho = s_A / (sqrt(m) s_y), the shared shift n (largest n <= 48 with
// every round(2^n rho) <= 32767) and M = round(2^n rho). Rows past d_out get
// zeros.
__global__ __launch_bounds__(256) void wh_constants_kernel(const float* __restrict__ bias,
                                                           const float* __restrict__ s_w,
                                                           int d_out, int d_out_pad, int m,
                                                           double s_x, double s_y,
                                                           int32_t* __restrict__ b_int,
                                                           int32_t* __restrict__ mult,
                                                           int32_t* __restrict__ shift) {
  __shared__ double red[256];
  const double sqm = sqrt(double(m));
  double top = 0.0;
  for (int c = threadIdx.x; c < d_out; c += 256) {
    const double rho = s_x * double(s_w[c]) / (sqm * s_y);
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
  int n = 0;
  if (top > 0.0)
    while (n < WH_SHIFT_MAX && rint(ldexp(top, n + 1)) <= double(WH_MULT_MAX)) ++n;
  if (threadIdx.x == 0) *shift = n;
  for (int c = threadIdx.x; c < d_out_pad; c += 256) {
    int32_t bi = 0, mc = 0;
    if (c < d_out) {
      const double s_a = s_x * double(s_w[c]);
      const double rho = s_a / (sqm * s_y);
      mc = int32_t(rint(ldexp(rho, n)));
      if (bias && s_a > 0.0) {
        const int base = (c / m) * m, ci = c - base;
        double bb = 0.0;
        for (int k = 0; k < m; ++k) {
          const double v = double(bias[base + k]);
          bb += (__popc(ci & k) & 1) ? -v : v;
        }
        double q = rint((bb / sqm) / s_a);
        q = q > double(WH_BIAS_MAX) ? double(WH_BIAS_MAX) : q;
        q = q < -double(WH_BIAS_MAX) ? -double(WH_BIAS_MAX) : q;
        bi = int32_t(q);
      }
    }
    b_int[c] = bi;
    mult[c] = mc;
  }
}

// round(v / 2^n), ties to even, for n >= 1.
__device__ __forceinline__ int64_t rne_shift(int64_t v, int n) {
  const int64_t q = v >> n;
  const int64_t r = v - (q << n);
  const int64_t half = int64_t(1) << (n - 1);
  return q + ((r > half || (r == half && (q & 1))) ? 1 : 0);
}

// Requantisation of int32 products acc [T, ldc] (without bias): one wave per
// (token, 256-channel chunk), lane l holding channels 4 l .. 4 l + 3 of the
// chunk. u = M (acc + b_int) in int64, the unnormalised Sylvester butterflies
// over blocks of m channels (channel bits 0-1 inside the lane, bits 2.. across
// lanes), then round(u / 2^n) with ties to even and clamping to +-127.
__global__ __launch_bounds__(256) void wh_requant_kernel(
    const int32_t* __restrict__ acc, int64_t ldc, int64_t T, int d_out, int chunks, int m,
    const int32_t* __restrict__ b_int, const int32_t* __restrict__ mult,
    const int32_t* __restrict__ shift, int8_t* __restrict__ y, int64_t ldy) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (unit >= T * chunks) return;   // whole waves leave together
  const int64_t row = unit / chunks;
  const int c = int(unit - row * chunks) * 256 + 4 * lane;
  const bool valid = c < d_out;     // d_out % 8 == 0: a lane is all in or all out
  int64_t u[4] = {0, 0, 0, 0};
  if (valid) {
    const int4 a = *reinterpret_cast<const int4*>(acc + row * ldc + c);
    const int4 b = *reinterpret_cast<const int4*>(b_int + c);
    const int4 mm = *reinterpret_cast<const int4*>(mult + c);
    u[0] = int64_t(mm.x) * int64_t(a.x + b.x);
    u[1] = int64_t(mm.y) * int64_t(a.y + b.y);
    u[2] = int64_t(mm.z) * int64_t(a.z + b.z);
    u[3] = int64_t(mm.w) * int64_t(a.w + b.w);
  }
  if (m >= 2) {
    const int64_t p0 = u[0] + u[1], q0 = u[0] - u[1], p1 = u[2] + u[3], q1 = u[2] - u[3];
    u[0] = p0; u[1] = q0; u[2] = p1; u[3] = q1;
  }
  if (m >= 4) {
    const int64_t p0 = u[0] + u[2], q0 = u[0] - u[2], p1 = u[1] + u[3], q1 = u[1] - u[3];
    u[0] = p0; u[2] = q0; u[1] = p1; u[3] = q1;
  }
  for (int dl = 1; 4 * dl < m; dl <<= 1) {
    const bool upper = (lane & dl) != 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int64_t o = __shfl_xor(u[k], dl);
      u[k] = upper ? o - u[k] : u[k] + o;
    }
  }
  if (!valid) return;
  const int n = *shift;
  uint32_t packed = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    int64_t q = n > 0 ? rne_shift(u[k], n) : u[k];
    q = q > 127 ? 127 : (q < -127 ? -127 : q);
    packed |= (uint32_t(q) & 0xFFu) << (8 * k);
  }
  *reinterpret_cast<uint32_t*>(y + row * ldy + c) = packed;
}

hipError_t launch_wh_weight(const void* w, int w_bf16, int d_out, int d_in, int m, float* wbar,
                            hipStream_t s) {
  if (m < 1 || m > WH_MAX_BLOCK || (m & (m - 1)) || d_out % m) return hipErrorInvalidValue;
  dim3 grid{unsigned((d_in + 31) / 32), unsigned(d_out / m)};
  const float ism = 1.0f / sqrtf(float(m));
  if (w_bf16)
    hipLaunchKernelGGL(wh_weight_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(w), d_in, m, ism, wbar);
  else
    hipLaunchKernelGGL(wh_weight_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(w), d_in, m, ism, wbar);
  return hipGetLastError();
}

hipError_t launch_wh_constants(const float* bias, const float* s_w, int d_out, int d_out_pad,
                               int m, float s_x, float s_y, int32_t* b_int, int32_t* mult,
                               int32_t* shift, hipStream_t s) {
  hipLaunchKernelGGL(wh_constants_kernel, dim3(1), dim3(256), 0, s, bias, s_w, d_out, d_out_pad,
                     m, double(s_x), double(s_y), b_int, mult, shift);
  return hipGetLastError();
}

hipError_t launch_wh_requant(const int32_t* acc, int64_t ldc, int64_t T, int d_out, int m,
                             const int32_t* b_int, const int32_t* mult, const int32_t* shift,
                             int8_t* y, int64_t ldy, hipStream_t s) {
  if (T <= 0) return hipSuccess;
  if (m < 1 || m > WH_MAX_BLOCK || (m & (m - 1)) || d_out % m || d_out % 8)
    return hipErrorInvalidValue;
  const int chunks = (d_out + 255) / 256;
  const int64_t waves = T * chunks;
  hipLaunchKernelGGL(wh_requant_kernel, dim3(unsigned((waves + 3) / 4)), dim3(256), 0, s, acc, ldc,
                     T, d_out, chunks, m, b_int, mult, shift, y, ldy);
  return hipGetLastError();
}

}  // namespace hq
