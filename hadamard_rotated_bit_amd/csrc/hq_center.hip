// Per-channel centring of libhq (descriptor center = 2): the other reading of
// HadaNorm Eq. (1) ("What carries the argument"; Fig. 2 caption: mu and sigma
// in R^d; "one added token"). mu is the mean over the T tokens of the call of
// each scaled-and-rotated channel, mu = (mean_t X) diag(1/sigma) H by
// linearity, and the correction mu W~ = (mean_t X) W is one bias vector for
// every token. On the GPU the mean is subtracted before the rotation,
// ((X - 1 m^T) diag(1/sigma), then H: the same X~), inside the row transform;
// these kernels produce m = mean_t X and the corrected bias.
#include "hq_device.h"
#include "hq_internal.h"

namespace hq {

// Partial column sums of X [rows, d] over chunks of `rpc` rows: block
// (x, y) sums columns [512 x, 512 x + 512) over rows [rpc y, rpc (y + 1)),
// 64 column lanes of 8 channels times 4 row lanes, the 4 row lanes combined
// in a fixed order. partial [chunks, d].
template <typename TIn>
__global__ __launch_bounds__(256) void col_partial_kernel(const TIn* __restrict__ in, int64_t rows,
                                                          int d, int64_t rpc,
                                                          float* __restrict__ partial) {
  const int cl = threadIdx.x & 63, rl = threadIdx.x >> 6;
  const int c0 = int(blockIdx.x) * 512 + cl * 8;
  const int64_t r0 = int64_t(blockIdx.y) * rpc;
  const int64_t r1 = (r0 + rpc) < rows ? (r0 + rpc) : rows;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (c0 < d) {
    for (int64_t r = r0 + rl; r < r1; r += 4) {
      float v[8];
      load8(in + r * d + c0, v);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] += v[j];
    }
  }
  __shared__ float red[4][512];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[rl][cl * 8 + j] = acc[j];
  __syncthreads();
  if (rl == 0 && c0 < d) {
    float out[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      out[j] = ((red[0][cl * 8 + j] + red[1][cl * 8 + j]) + red[2][cl * 8 + j]) + red[3][cl * 8 + j];
    float* o = partial + int64_t(blockIdx.y) * d + c0;
    reinterpret_cast<float4*>(o)[0] = make_float4(out[0], out[1], out[2], out[3]);
    reinterpret_cast<float4*>(o)[1] = make_float4(out[4], out[5], out[6], out[7]);
  }
}

// mean[i] = (sum of the chunk partials) / rows. Block: 64 columns x 4 chunk
// lanes; lane g sums chunks g, g + 4, ... eight loads at a time (issued
// together, added as a fixed tree), and the 4 lane sums are combined in lane
// order, so the result does not depend on timing.
__global__ __launch_bounds__(256) void mean_finish_kernel(const float* __restrict__ partial,
                                                          int chunks, int64_t rows, int d,
                                                          float* __restrict__ mean) {
  const int ci = threadIdx.x & 63, g = threadIdx.x >> 6;
  const int i = int(blockIdx.x) * 64 + ci;
  float s = 0.0f;
  if (i < d) {
    int c = g;
    for (; c + 28 < chunks; c += 32) {
      float p[8];
#pragma unroll
      for (int k = 0; k < 8; ++k) p[k] = partial[int64_t(c + 4 * k) * d + i];
      s += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    }
    for (; c < chunks; c += 4) s += partial[int64_t(c) * d + i];
  }
  __shared__ float red[4][64];
  red[g][ci] = s;
  __syncthreads();
  if (g == 0 && i < d)
    mean[i] = (((red[0][ci] + red[1][ci]) + red[2][ci]) + red[3][ci]) / float(rows);
}

// out[j] = bias[j] + sum_i weight[j, i] mean[i] for j < n (the corrected bias
// b + mu W~ = b + (mean_t X) W), out[j] = bias[j] for n <= j < n_pad. One
// wave per output row, fp32 accumulation in a fixed order.
template <typename TW>
__global__ __launch_bounds__(256) void bias_gemv_kernel(const TW* __restrict__ weight,
                                                        const float* __restrict__ mean,
                                                        const float* __restrict__ bias, int n,
                                                        int n_pad, int d, float* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int j = int(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (j >= n_pad) return;
  float acc = 0.0f;
  if (j < n) {
    const TW* w = weight + int64_t(j) * d;
    for (int i0 = lane * 8; i0 < d; i0 += 512) {
      float wv[8], mv[8];
      load8(w + i0, wv);
      load8(mean + i0, mv);
#pragma unroll
      for (int k = 0; k < 8; ++k) acc = fmaf(wv[k], mv[k], acc);
    }
  }
  acc = group_sum<64>(acc);
  if (lane == 0) out[j] = bias[j] + acc;
}

int center_chunks(int64_t rows) { return int((rows + CENTER_RPC - 1) / CENTER_RPC); }

hipError_t launch_channel_mean(const void* x, int x_bf16, int64_t rows, int d, float* partial,
                               float* mean, hipStream_t s) {
  if (rows <= 0) return hipErrorInvalidValue;
  const int chunks = center_chunks(rows);
  const dim3 grid{unsigned((d + 511) / 512), unsigned(chunks)};
  if (x_bf16)
    hipLaunchKernelGGL(col_partial_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(x), rows, d, int64_t(CENTER_RPC), partial);
  else
    hipLaunchKernelGGL(col_partial_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(x), rows, d, int64_t(CENTER_RPC), partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mean_finish_kernel, dim3((d + 63) / 64), dim3(256), 0, s, partial, chunks,
                     rows, d, mean);
  return hipGetLastError();
}

hipError_t launch_bias_gemv(const void* weight, int w_bf16, const float* mean, const float* bias,
                            int n, int n_pad, int d, float* out, hipStream_t s) {
  const dim3 grid{unsigned((n_pad + 3) / 4)};
  if (w_bf16)
    hipLaunchKernelGGL(bias_gemv_kernel<uint16_t>, grid, dim3(256), 0, s,
                       static_cast<const uint16_t*>(weight), mean, bias, n, n_pad, d, out);
  else
    hipLaunchKernelGGL(bias_gemv_kernel<float>, grid, dim3(256), 0, s,
                       static_cast<const float*>(weight), mean, bias, n, n_pad, d, out);
  return hipGetLastError();
}

}  // namespace hq
