// CPU oracle in plain C++17 for the rotated-and-centred quantised linear
// layer: the same definitions as oracle/hq_oracle.py, written out directly,
// with std::thread over rows.
//
// TEST INFRASTRUCTURE ONLY. Nothing in the library's product path may load
// or call this code: the tests, the entry point's smoke check and the
// benchmark's CPU-baseline leg use it, nothing else. It shares no code with
// the HIP path (no kernels, helpers, tables or constants) and includes
// nothing of it.
//
// Sources (page titles; equations as numbered there):
//  * HadaNorm review ("What carries the argument"), Eq. (1):
//    X W + b = X~ W~ + b~, X~ = X diag(1/sigma) H - mu, W~ = H^T diag(sigma) W,
//    b~ = b + mu W~, mu the per-token mean of X diag(1/sigma) H.
//  * HaTQ ("Hadamard-Domain Model Quantization for Learned Image Coding"):
//    Sec. III-A Eq. (3) the symmetric quantiser, Sec. III-B Eq. (4) the
//    integer product, Sec. III-C Eq. (8) the Hadamard transform as signed
//    sums, supplement Sec. VII-A the Sylvester matrix, Eq. (18) the
//    accumulator scale s_x s_w.
//  * Data-free int4 blog ("Hadamard rotation: the int4 improvement", steps
//    3-4 and 7): block-diagonal rotation over contiguous channel blocks, the
//    16-bit low-rank branch on the smoothed, un-rotated input.
//
// Every floating-point step is float64. Readings (the same as the Python
// oracle): H is the normalised Sylvester matrix, entry (i, j) =
// (-1)^popcount(i & j) / sqrt(B), applied per block of B contiguous
// channels; round() is half to even; a row whose maximum is 0 gets scale 0
// and zero codes; c = 1^T W~ from the unquantised W~; mu is one scalar per
// token (center = 1) or 0 (center = 0). Centring over channels and
// group-wise scales are covered by the Python oracle only.
//
// Integer products: codes are at most 127 in magnitude and d_in at most
// 8192, so every partial sum of code products is below 127^2 * 8192 < 2^31
// and int32 accumulation is exact (checked); the sums are returned as int64.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>

namespace {

// Runs f(begin, end) over [0, n) split into `threads` contiguous ranges.
template <typename F>
void parallel_rows(int64_t n, int threads, F f) {
  if (threads < 1) threads = 1;
  if (n < threads) threads = int(n > 0 ? n : 1);
  std::vector<std::thread> pool;
  const int64_t per = (n + threads - 1) / threads;
  for (int k = 0; k < threads; ++k) {
    const int64_t b = k * per, e = b + per < n ? b + per : n;
    if (b >= e) break;
    pool.emplace_back([=]() { f(b, e); });
  }
  for (auto& t : pool) t.join();
}

int popcount(unsigned v) {
  int c = 0;
  for (; v; v &= v - 1) ++c;
  return c;
}

// Sylvester sign matrix of order B: sgn[i * B + j] = (-1)^popcount(i & j).
std::vector<signed char> sylvester_signs(int B) {
  std::vector<signed char> s(size_t(B) * B);
  for (int i = 0; i < B; ++i)
    for (int j = 0; j < B; ++j) s[size_t(i) * B + j] = (popcount(unsigned(i & j)) & 1) ? -1 : 1;
  return s;
}

// y = x diag(H_B, ..., H_B) for one row of d channels: each output of a block
// is the normalised signed sum of the block's inputs (HaTQ Eq. (8)).
void rotate_row(const double* x, int d, int B, const signed char* sgn, double* y) {
  const double nrm = 1.0 / std::sqrt(double(B));
  for (int k0 = 0; k0 < d; k0 += B)
    for (int j = 0; j < B; ++j) {
      double acc = 0.0;
      for (int i = 0; i < B; ++i) acc += sgn[size_t(i) * B + j] * x[k0 + i];
      y[k0 + j] = acc * nrm;
    }
}

// Symmetric quantiser of one row (HaTQ Eq. (3)): s = max|v| / qmax,
// q = clamp(round(v / s), -qmax, qmax), round half to even (nearbyint under
// the default rounding mode).
void quantize_row(const double* v, int n, int qmax, int16_t* q, double* s_out) {
  double amax = 0.0;
  for (int i = 0; i < n; ++i) amax = std::fabs(v[i]) > amax ? std::fabs(v[i]) : amax;
  const double s = amax / qmax;
  *s_out = s;
  for (int i = 0; i < n; ++i) {
    double t = s > 0.0 ? std::nearbyint(v[i] / s) : 0.0;
    if (t > qmax) t = qmax;
    if (t < -qmax) t = -qmax;
    q[i] = int16_t(t);
  }
}

// float64 -> nearest bf16 value (ties to even), returned as float64.
double round_bf16(double y) {
  if (y == 0.0 || !std::isfinite(y)) return y;
  int e;
  const double m = std::frexp(y, &e);            // y = m 2^e, 0.5 <= |m| < 1
  return std::ldexp(std::nearbyint(std::ldexp(m, 8)), e - 8);   // 8 significant bits
}

}  // namespace

extern "C" {

// Offline half (HadaNorm Eq. (1) weight side): row j of W~^T is
// (weight_j * sigma) H; c_j = sum_i W~_ji; codes and s_w per output channel.
//  weight [d_out, d_in], sigma [d_in] (NULL = ones). Outputs qw [d_out, d_in],
//  s_w [d_out], c [d_out]. Returns 0, or -1 on a bad argument.
int hqo_prepare(int d_in, int d_out, int block, int w_bits, const double* weight,
                const double* sigma, int16_t* qw, double* s_w, double* c, int threads) {
  if (d_in <= 0 || d_out <= 0 || block <= 0 || d_in % block || (block & (block - 1)) ||
      (w_bits != 4 && w_bits != 8))
    return -1;
  const std::vector<signed char> sgn = sylvester_signs(block);
  const int qmax = (1 << (w_bits - 1)) - 1;
  parallel_rows(d_out, threads, [&](int64_t b, int64_t e) {
    std::vector<double> v(d_in), wt(d_in);
    for (int64_t j = b; j < e; ++j) {
      for (int i = 0; i < d_in; ++i)
        v[i] = weight[j * d_in + i] * (sigma ? sigma[i] : 1.0);
      rotate_row(v.data(), d_in, block, sgn.data(), wt.data());
      double cs = 0.0;
      for (int i = 0; i < d_in; ++i) cs += wt[i];
      c[j] = cs;
      quantize_row(wt.data(), d_in, qmax, qw + j * d_in, &s_w[j]);
    }
  });
  return 0;
}

// Online half for T tokens: x' = x / sigma, y = x' H, mu (center = 1) and
// x~ = y - mu, per-token codes and s_x, the integer product with the weight
// codes, and Y = s_x s_w acc + b + mu c (+ (x' L1) L2), rounded once to the
// output type (out_bf16 = 1: bf16, else fp32).
//  x [T, d_in]; sigma [d_in] or NULL; qw [d_out, d_in], s_w, c [d_out]
//  (from hqo_prepare); bias [d_out] or NULL; l1 [d_in, rank], l2 [rank, d_out]
//  (rank 0: NULL). Outputs: qa [T, d_in], s_x [T], mu [T], acc [T, d_out]
//  (NULL: not returned), y [T, d_out]. Returns 0, -1 on a bad argument, -2
//  if a partial sum would leave the exact int32 range.
int hqo_quant_linear(int64_t T, int d_in, int d_out, int block, int a_bits, int center,
                     const double* x, const double* sigma, const int16_t* qw, const double* s_w,
                     const double* c, const double* bias, int rank, const double* l1,
                     const double* l2, int out_bf16, int16_t* qa, double* s_x, double* mu,
                     int64_t* acc, double* y, int threads) {
  if (T < 0 || d_in <= 0 || d_out <= 0 || block <= 0 || d_in % block ||
      (block & (block - 1)) || (a_bits != 4 && a_bits != 8) || (center != 0 && center != 1) ||
      rank < 0 || (rank && (!l1 || !l2)))
    return -1;
  int wmax = 0;
  for (int64_t i = 0; i < int64_t(d_out) * d_in; ++i)
    wmax = std::abs(int(qw[i])) > wmax ? std::abs(int(qw[i])) : wmax;
  const int qmax = (1 << (a_bits - 1)) - 1;
  if (double(qmax) * wmax * d_in >= 2147483648.0) return -2;
  const std::vector<signed char> sgn = sylvester_signs(block);
  parallel_rows(T, threads, [&](int64_t b, int64_t e) {
    std::vector<double> xp(d_in), yr(d_in), u(rank > 0 ? rank : 1);
    for (int64_t t = b; t < e; ++t) {
      for (int i = 0; i < d_in; ++i) xp[i] = x[t * d_in + i] / (sigma ? sigma[i] : 1.0);
      rotate_row(xp.data(), d_in, block, sgn.data(), yr.data());
      double m = 0.0;
      if (center) {
        for (int i = 0; i < d_in; ++i) m += yr[i];
        m /= d_in;
        for (int i = 0; i < d_in; ++i) yr[i] -= m;
      }
      mu[t] = m;
      int16_t* q = qa + t * d_in;
      quantize_row(yr.data(), d_in, qmax, q, &s_x[t]);
      for (int k = 0; k < rank; ++k) {
        double s = 0.0;
        for (int i = 0; i < d_in; ++i) s += xp[i] * l1[int64_t(i) * rank + k];
        u[k] = s;
      }
      for (int j = 0; j < d_out; ++j) {
        const int16_t* w = qw + int64_t(j) * d_in;
        int32_t a = 0;
        for (int i = 0; i < d_in; ++i) a += int32_t(q[i]) * int32_t(w[i]);
        if (acc) acc[t * d_out + j] = a;
        double v = s_x[t] * s_w[j] * double(a) + (bias ? bias[j] : 0.0) + m * c[j];
        if (rank) {
          double lr = 0.0;
          for (int k = 0; k < rank; ++k) lr += u[k] * l2[int64_t(k) * d_out + j];
          v += lr;
        }
        y[t * d_out + j] = out_bf16 ? round_bf16(v) : double(float(v));
      }
    }
  });
  return 0;
}

// The rotation alone (for the pins): out = in diag(H_B, ...) row by row.
int hqo_rotate(int64_t rows, int d, int block, const double* in, double* out) {
  if (rows < 0 || d <= 0 || block <= 0 || d % block || (block & (block - 1))) return -1;
  const std::vector<signed char> sgn = sylvester_signs(block);
  for (int64_t r = 0; r < rows; ++r) rotate_row(in + r * d, d, block, sgn.data(), out + r * d);
  return 0;
}

}  // extern "C"
