// C ABI of libhq: host-side validation, buffer layout and kernel dispatch.
// Every check runs on the host before anything is enqueued; the library never
// allocates device memory.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "../../include/hq.h"
#include "hq_internal.h"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(HQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr uint32_t kMagic = 0x31505148u;  // "HQP1"

struct PreparedHeader {
  uint32_t magic;
  uint32_t version;
  hq_desc desc;
  int64_t d_out_pad;
  uint64_t total;
};
static_assert(sizeof(PreparedHeader) <= 256, "header fits in 256 bytes");

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline bool is_pow2(int v) { return v > 0 && (v & (v - 1)) == 0; }
inline int log2i(int v) {
  int l = 0;
  while ((1 << l) < v) ++l;
  return l;
}
inline float qmax_of(int bits) { return float((1 << (bits - 1)) - 1); }
// Scales per row: 1, or one per 64-channel group.
inline int64_t scales_per_row(const hq_desc* d) { return d->group ? d->d_in / d->group : 1; }

int check_desc(const hq_desc* d) {
  if (!d) return fail(HQ_ERR_INVALID_ARG, "desc is NULL");
  if (d->d_in <= 0 || d->d_out <= 0)
    return fail(HQ_ERR_INVALID_ARG, "d_in and d_out must be positive (got %d, %d)", d->d_in,
                d->d_out);
  if (d->x_dtype != HQ_F32 && d->x_dtype != HQ_BF16)
    return fail(HQ_ERR_INVALID_ARG, "x_dtype %d is not an hq_dtype", d->x_dtype);
  if (d->w_dtype != HQ_F32 && d->w_dtype != HQ_BF16)
    return fail(HQ_ERR_INVALID_ARG, "w_dtype %d is not an hq_dtype", d->w_dtype);
  if (d->y_dtype != HQ_F32 && d->y_dtype != HQ_BF16)
    return fail(HQ_ERR_INVALID_ARG, "y_dtype %d is not an hq_dtype", d->y_dtype);
  if (d->gemm != HQ_GEMM_AUTO && d->gemm != HQ_GEMM_I8)
    return fail(HQ_ERR_INVALID_ARG, "gemm %d is not an hq_gemm_engine", d->gemm);
  if (d->center != HQ_CENTER_NONE && d->center != HQ_CENTER_TOKEN && d->center != HQ_CENTER_CHANNEL)
    return fail(HQ_ERR_INVALID_ARG, "center must be 0, 1 or 2 (got %d)", d->center);
  if (d->smooth != 0 && d->smooth != 1)
    return fail(HQ_ERR_INVALID_ARG, "smooth must be 0 or 1 (got %d)", d->smooth);
  if (d->a_bits != 4 && d->a_bits != 8)
    return fail(HQ_ERR_UNSUPPORTED, "a_bits must be 4 or 8 (got %d)", d->a_bits);
  if (d->w_bits != 4 && d->w_bits != 8)
    return fail(HQ_ERR_UNSUPPORTED, "w_bits must be 4 or 8 (got %d)", d->w_bits);
  hq::RowGeom g;
  if (d->d_in % 128 || !hq::row_geometry(d->d_in, &g))
    return fail(HQ_ERR_UNSUPPORTED,
                "d_in %d unsupported: need a multiple of 128 up to 2048, of 256 up to 4096, or "
                "of 512 up to 8192",
                d->d_in);
  if (d->d_out % 8)
    return fail(HQ_ERR_UNSUPPORTED, "d_out must be a multiple of 8 (got %d)", d->d_out);
  if (!is_pow2(d->block) || d->d_in % d->block)
    return fail(HQ_ERR_UNSUPPORTED, "block %d must be a power of two dividing d_in %d", d->block,
                d->d_in);
  if (d->rank < 0 || d->rank > 64 || d->rank % 16)
    return fail(HQ_ERR_UNSUPPORTED, "rank must be 0, 16, 32, 48 or 64 (got %d)", d->rank);
  if (d->group != 0 && d->group != 64)
    return fail(HQ_ERR_UNSUPPORTED, "group must be 0 or 64 (got %d)", d->group);
  if (d->group && (d->a_bits != 4 || d->w_bits != 4 || d->gemm != HQ_GEMM_AUTO))
    return fail(HQ_ERR_UNSUPPORTED,
                "group = 64 needs a_bits = w_bits = 4 and gemm = HQ_GEMM_AUTO (FP6 engine)");
  return HQ_OK;
}

bool misaligned(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) != 0; }

// Both operands use E2M3 (FP6 MFMA) when both code widths are 4 bits and the
// engine is automatic, else int8 bytes (int8 MFMA).
int code_fmt_of(const hq_desc* d) {
  return (d->gemm == HQ_GEMM_AUTO && d->a_bits == 4 && d->w_bits == 4) ? hq::CODES_E2M3
                                                                         : hq::CODES_I8;
}

void layout_of(const hq_desc* d, hq_prepared_layout* L) {
  const int64_t np = round_up(d->d_out, hq::GEMM_BN);
  size_t off = 256;
  L->d_out_pad = np;
  L->w_codes = off;
  off += align256(hq::code_bytes(code_fmt_of(d), np, d->d_in));
  L->w_scale = off;
  off += align256(4 * size_t(np) * scales_per_row(d));
  L->c = off;
  off += align256(4 * size_t(np));
  L->bias = off;
  off += align256(4 * size_t(np));
  L->sigma_inv = off;
  off += align256(4 * size_t(d->d_in));
  L->l1_hi = off;
  off += align256(2 * size_t(d->rank) * d->d_in);
  L->l1_lo = off;
  off += align256(2 * size_t(d->rank) * d->d_in);
  L->l2_hi = off;
  off += align256(2 * size_t(np) * d->rank);
  L->l2_lo = off;
  off += align256(2 * size_t(np) * d->rank);
  L->weight = 0;
  if (d->center == HQ_CENTER_CHANNEL) {
    L->weight = off;
    off += align256(size_t(d->w_dtype == HQ_BF16 ? 2 : 4) * size_t(d->d_out) * d->d_in);
  }
  L->total = off;
}

struct Workspace {
  size_t codes, s_x, mu, U;
  size_t lr_part;                  // rank > 0 with the split down projection
  size_t partial, mean, bias_eff;  // center = 2 only
  size_t total;
};
Workspace workspace_of(const hq_desc* d, int64_t T) {
  Workspace w = {};
  size_t off = 0;
  w.codes = off;
  off += align256(hq::code_bytes(code_fmt_of(d), T, d->d_in));
  w.s_x = off;
  off += align256(4 * size_t(T) * scales_per_row(d));
  w.mu = off;
  off += align256(4 * size_t(T));
  w.U = off;
  off += align256(4 * size_t(T) * d->rank);
  const int ks = d->rank ? hq::lowrank_slices(d->d_in, d->rank, T) : 0;
  w.lr_part = ks ? off : 0;
  off += align256(4 * size_t(ks) * size_t(T) * d->rank);
  if (d->center == HQ_CENTER_CHANNEL) {
    w.partial = off;
    off += align256(4 * size_t(hq::center_chunks(T > 0 ? T : 1)) * d->d_in);
    w.mean = off;
    off += align256(4 * size_t(d->d_in));
    w.bias_eff = off;
    off += align256(4 * size_t(round_up(d->d_out, hq::GEMM_BN)));
  }
  w.total = off;
  return w;
}

template <typename P>
inline P* at(void* base, size_t off) {
  return reinterpret_cast<P*>(static_cast<uint8_t*>(base) + off);
}
template <typename P>
inline const P* at(const void* base, size_t off) {
  return reinterpret_cast<const P*>(static_cast<const uint8_t*>(base) + off);
}

// Per-channel centring statistics of the T rows of X (center = 2): mean
// [d_in] = mean_t X, subtracted by the row transform, and bias_eff
// [d_out_pad] = b + weight . mean, the corrected bias of the GEMM epilogue.
int run_center(const hq_desc* d, const void* prepared, const void* X, int64_t T, float* partial,
               float* mean, float* bias_eff, hipStream_t s) {
  hq_prepared_layout L;
  layout_of(d, &L);
  hipError_t e = hq::launch_channel_mean(X, d->x_dtype == HQ_BF16, T, d->d_in, partial, mean, s);
  if (e == hipSuccess)
    e = hq::launch_bias_gemv(at<uint8_t>(prepared, L.weight), d->w_dtype == HQ_BF16, mean,
                             at<float>(prepared, L.bias), d->d_out, int(L.d_out_pad), d->d_in,
                             bias_eff, s);
  return e == hipSuccess ? HQ_OK : hip_fail(e, "centring kernel launch");
}

// Activation stage shared by hq_quant_linear and hq_act_quantize. For
// center = 2, `cmean` is the per-channel mean and `mu` (per-token) is NULL;
// otherwise cmean is NULL and mu gets the per-token means.
int run_act(const hq_desc* d, const void* prepared, const void* X, int64_t T, void* codes,
            float* s_x, float* mu, const float* cmean, float* U, hipStream_t s,
            float* lr_part = nullptr) {
  hq_prepared_layout L;
  layout_of(d, &L);
  hq::RowArgs a = {};
  a.in = X;
  a.in_bf16 = d->x_dtype == HQ_BF16;
  a.rows = T;
  a.d = d->d_in;
  // with per-channel centring the multipliers are always passed (the blob
  // holds ones without smoothing): the fast row kernel takes means only
  // together with multipliers
  a.scale = (d->smooth || cmean) ? at<float>(prepared, L.sigma_inv) : nullptr;
  a.chan_mean = cmean;
  a.log2b = log2i(d->block);
  a.center = d->center == HQ_CENTER_TOKEN;
  a.qmax = qmax_of(d->a_bits);
  a.codes = static_cast<uint8_t*>(codes);
  a.code_fmt = code_fmt_of(d);
  a.out_s = s_x;
  a.group = d->group;
  a.s_ld = T;
  a.out_aux = mu;
  a.mode = hq::ROW_ACT;
  hq::RowGeom g;
  if (d->rank && hq::row_geometry(d->d_in, &g) && hq::act_lr_applies(a, g, d->rank)) {
    // row transform and low-rank projection in one launch
    const hipError_t e = hq::launch_act_lr(a, g, d->rank, at<uint16_t>(prepared, L.l1_hi),
                                           at<uint16_t>(prepared, L.l1_lo), U, s);
    return e == hipSuccess ? HQ_OK : hip_fail(e, "activation kernel launch");
  }
  hipError_t e = hq::launch_row_transform(a, s);
  if (e != hipSuccess) return hip_fail(e, "activation kernel launch");
  if (d->rank) {
    // with a workspace for the slice products: the split form (same U bits)
    if (lr_part)
      e = hq::launch_lowrank_split(X, a.in_bf16, T, d->d_in, d->rank,
                                   at<uint16_t>(prepared, L.l1_hi),
                                   at<uint16_t>(prepared, L.l1_lo), lr_part, U, s);
    else
      e = hq::launch_lowrank_down(X, a.in_bf16, T, d->d_in, d->rank,
                                  at<uint16_t>(prepared, L.l1_hi),
                                  at<uint16_t>(prepared, L.l1_lo), U, s);
    if (e != hipSuccess) return hip_fail(e, "low-rank kernel launch");
  }
  return HQ_OK;
}

// Integer GEMM on the descriptor's code format.
hipError_t launch_codes_gemm(const hq_desc* d, const void* a_codes, int64_t T, const void* w_codes,
                             int64_t N, int32_t* acc, int64_t ldc, const hq::GemmEpi* ep,
                             hipStream_t s) {
  if (code_fmt_of(d) == hq::CODES_E2M3)
    return hq::launch_gemm_f6(static_cast<const uint8_t*>(a_codes), T,
                              static_cast<const uint8_t*>(w_codes), N, d->d_in, acc, ldc, ep, s);
  return hq::launch_gemm(static_cast<const int8_t*>(a_codes), T,
                         static_cast<const int8_t*>(w_codes), N, d->d_in, acc, ldc, ep, s);
}

// GEMM + epilogue. For center = 2 `mu` is the corrected bias [d_out_pad]
// (b + weight . mean) and replaces b; the prepared c is zero in that mode, so
// the per-token term vanishes (s_x stands in for the per-token vector).
int run_gemm_dequant(const hq_desc* d, const void* prepared, const void* codes,
                     const float* s_x, const float* mu, const float* U, int64_t T, void* Y,
                     hipStream_t s) {
  hq_prepared_layout L;
  layout_of(d, &L);
  const bool chan = d->center == HQ_CENTER_CHANNEL;
  hq::GemmEpi ep = {};
  ep.s_x = s_x;
  ep.mu = chan ? s_x : mu;
  ep.s_w = at<float>(prepared, L.w_scale);
  ep.c = at<float>(prepared, L.c);
  ep.bias = chan ? mu : at<float>(prepared, L.bias);
  ep.U = U;
  ep.l2_hi = at<uint16_t>(prepared, L.l2_hi);
  ep.l2_lo = at<uint16_t>(prepared, L.l2_lo);
  // L2 given in bf16 is exactly its bf16 hi part: the lo part is all zero
  ep.l2_lo_zero = d->w_dtype == HQ_BF16;
  ep.rank = d->rank;
  ep.Y = Y;
  ep.y_bf16 = d->y_dtype == HQ_BF16;
  ep.ldy = d->d_out;
  hipError_t e =
      d->group ? hq::launch_gemm_f6g(static_cast<const uint8_t*>(codes), T,
                                     at<uint8_t>(prepared, L.w_codes), d->d_out, d->d_in, s_x, T,
                                     ep.s_w, L.d_out_pad, &ep, s)
               : launch_codes_gemm(d, codes, T, at<uint8_t>(prepared, L.w_codes), d->d_out,
                                   nullptr, 0, &ep, s);
  if (e != hipSuccess) return hip_fail(e, "GEMM kernel launch");
  return HQ_OK;
}

// ---- integer-only DH / WH layers ---------------------------------------------

constexpr uint32_t kMagicInt = 0x31495148u;  // "HQI1"

struct IntHeader {
  uint32_t magic;
  uint32_t version;
  hq_int_desc desc;
  int64_t d_out_pad;
  uint64_t total;
  float s_x, s_y, s_z, s_u;
};
static_assert(sizeof(IntHeader) <= 256, "header fits in 256 bytes");

// Widths of an integer layer (padded orders, supplement Sec. VII-B): the
// input codes (a DH layer with in_block above d_in takes in_block of them),
// the accumulator channels (a WH layer with block above d_out has block of
// them) and the output codes (post_block above d_out: post_block of them).
int int_x_width(const hq_int_desc* d) {
  return d->side == HQ_INT_DH && d->in_block > d->d_in ? d->in_block : d->d_in;
}
int int_acc_width(const hq_int_desc* d) {
  return d->side == HQ_INT_WH && d->block > d->d_out ? d->block : d->d_out;
}
int int_out_width(const hq_int_desc* d) {
  return d->post_block > d->d_out ? d->post_block : d->d_out;
}

int check_int_desc(const hq_int_desc* d) {
  if (!d) return fail(HQ_ERR_INVALID_ARG, "desc is NULL");
  if (d->d_in <= 0 || d->d_out <= 0)
    return fail(HQ_ERR_INVALID_ARG, "d_in and d_out must be positive (got %d, %d)", d->d_in,
                d->d_out);
  if (d->w_dtype != HQ_F32 && d->w_dtype != HQ_BF16)
    return fail(HQ_ERR_INVALID_ARG, "w_dtype %d is not an hq_dtype", d->w_dtype);
  if (d->side != HQ_INT_WH && d->side != HQ_INT_DH)
    return fail(HQ_ERR_INVALID_ARG, "side must be HQ_INT_WH or HQ_INT_DH (got %d)", d->side);
  if (d->side == HQ_INT_WH && d->in_block != 1)
    return fail(HQ_ERR_UNSUPPORTED, "a WH layer takes in_block = 1 (got %d)", d->in_block);
  if (d->side == HQ_INT_DH &&
      (!is_pow2(d->in_block) || (d->d_in % d->in_block && d->in_block < d->d_in)))
    return fail(HQ_ERR_UNSUPPORTED,
                "in_block %d must be a power of two dividing d_in %d or above it (padded)",
                d->in_block, d->d_in);
  const int xw = int_x_width(d);
  hq::RowGeom g;
  if (xw % 128 || !hq::row_geometry(xw, &g))
    return fail(HQ_ERR_UNSUPPORTED,
                "input width %d unsupported: need a multiple of 128 up to 2048, of 256 up to "
                "4096, or of 512 up to 8192",
                xw);
  if (d->d_out % 8)
    return fail(HQ_ERR_UNSUPPORTED, "d_out must be a multiple of 8 (got %d)", d->d_out);
  if (!is_pow2(d->block) || d->block > hq::WH_MAX_BLOCK ||
      (d->d_out % d->block && (d->side == HQ_INT_DH || d->block < d->d_out)))
    return fail(HQ_ERR_UNSUPPORTED,
                "block %d must be a power of two <= %d dividing d_out %d (or above it for a "
                "padded WH order)",
                d->block, hq::WH_MAX_BLOCK, d->d_out);
  if (d->act < HQ_INT_ACT_NONE || d->act > HQ_INT_ACT_GELU)
    return fail(HQ_ERR_INVALID_ARG, "act %d is not an hq_int_act", d->act);
  if (!is_pow2(d->post_block) || d->post_block > hq::WH_MAX_BLOCK ||
      (d->d_out % d->post_block && d->post_block < d->d_out))
    return fail(HQ_ERR_UNSUPPORTED,
                "post_block %d must be a power of two <= %d dividing d_out %d or above it",
                d->post_block, hq::WH_MAX_BLOCK, d->d_out);
  if (d->side == HQ_INT_DH && d->act != HQ_INT_ACT_NONE && d->block != 1)
    return fail(HQ_ERR_UNSUPPORTED,
                "a DH layer has no output-side transform before its activation: put the next "
                "layer's H_in order in post_block and use block = 1 (got block %d)", d->block);
  return HQ_OK;
}

void int_layout_of(const hq_int_desc* d, hq_int_layout* L) {
  const int64_t np = round_up(int_acc_width(d), hq::GEMM_BN);
  const size_t xw = size_t(int_x_width(d));
  size_t off = 256;
  L->d_out_pad = np;
  L->w_codes = off;
  off += align256(size_t(np) * xw);
  L->w_scale = off;
  off += align256(4 * size_t(np));
  L->b_int = off;
  off += align256(4 * size_t(np));
  L->mult = off;
  off += align256(4 * size_t(np));
  L->shift = off;
  L->mult_in = off + 4;
  L->shift_in = off + 8;
  off += 256;
  L->lut = off;
  off += 256;
  L->wbar = off;
  off += align256(4 * size_t(int_acc_width(d)) * xw);
  L->total = off;
}

// The transition's constants inside a prepared blob.
hq::IntTransition transition_of(const hq_int_desc* d, const void* prepared) {
  hq_int_layout L;
  int_layout_of(d, &L);
  hq::IntTransition tr = {};
  tr.m = d->block;
  tr.post = d->post_block;
  tr.keep = d->d_out;
  tr.act = d->act == HQ_INT_ACT_SILU || d->act == HQ_INT_ACT_GELU ? 2 : d->act;
  tr.b_int = at<int32_t>(prepared, L.b_int);
  tr.mult = at<int32_t>(prepared, L.mult);
  tr.shift = at<int32_t>(prepared, L.shift);
  tr.lut = at<int8_t>(prepared, L.lut);
  tr.mult_in = at<int32_t>(prepared, L.mult_in);
  tr.shift_in = at<int32_t>(prepared, L.shift_in);
  return tr;
}

int run_int_requant(const hq_int_desc* d, const void* prepared, const int32_t* acc, int64_t T,
                    int8_t* y, hipStream_t s) {
  const int aw = int_acc_width(d), ow = int_out_width(d);
  hipError_t e = hq::launch_int_requant(acc, aw, T, aw, ow, transition_of(d, prepared), y, ow, s);
  return e == hipSuccess ? HQ_OK : hip_fail(e, "requantisation kernel launch");
}

}  // namespace

int hq::set_error(int code, const char* msg) { return fail(code, "%s", msg); }

extern "C" {

int hq_abi_version(void) { return HQ_ABI_VERSION; }

const char* hq_last_error(void) { return g_err.c_str(); }

const char* hq_status_str(int status) {
  switch (status) {
    case HQ_OK: return "HQ_OK";
    case HQ_ERR_INVALID_ARG: return "HQ_ERR_INVALID_ARG";
    case HQ_ERR_UNSUPPORTED: return "HQ_ERR_UNSUPPORTED";
    case HQ_ERR_WORKSPACE: return "HQ_ERR_WORKSPACE";
    case HQ_ERR_BAD_PREPARED: return "HQ_ERR_BAD_PREPARED";
    case HQ_ERR_HIP: return "HQ_ERR_HIP";
    default: return "HQ_ERR_UNKNOWN";
  }
}

int hq_validate(const hq_desc* desc) {
  g_err.clear();
  return check_desc(desc);
}

size_t hq_prepared_bytes(const hq_desc* desc) {
  g_err.clear();
  if (check_desc(desc) != HQ_OK) return 0;
  hq_prepared_layout L;
  layout_of(desc, &L);
  return L.total;
}

int hq_prepared_layout_of(const hq_desc* desc, hq_prepared_layout* out) {
  g_err.clear();
  if (!out) return fail(HQ_ERR_INVALID_ARG, "out is NULL");
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  layout_of(desc, out);
  return HQ_OK;
}

size_t hq_workspace_bytes(const hq_desc* desc, int64_t T) {
  g_err.clear();
  if (check_desc(desc) != HQ_OK) return 0;
  if (T < 0) {
    fail(HQ_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
    return 0;
  }
  return workspace_of(desc, T).total;
}

int hq_code_format(const hq_desc* desc) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  return code_fmt_of(desc);
}

size_t hq_code_bytes(const hq_desc* desc, int64_t rows) {
  g_err.clear();
  if (check_desc(desc) != HQ_OK) return 0;
  if (rows < 0) {
    fail(HQ_ERR_INVALID_ARG, "rows must be >= 0 (got %lld)", (long long)rows);
    return 0;
  }
  return hq::code_bytes(code_fmt_of(desc), rows, desc->d_in);
}

int hq_channel_absmax(const hq_desc* desc, const void* X, int64_t T, float* absmax,
                      void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 0");
  if (!absmax || (T > 0 && !X)) return fail(HQ_ERR_INVALID_ARG, "X or absmax is NULL");
  if (misaligned(X) || misaligned(absmax))
    return fail(HQ_ERR_INVALID_ARG, "X and absmax must be 16-byte aligned");
  hipError_t e = hq::launch_col_absmax(X, desc->x_dtype == HQ_BF16, T, desc->d_in, absmax,
                                       static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HQ_OK : hip_fail(e, "absmax kernel launch");
}

int hq_sigma(const hq_desc* desc, const float* act_absmax, const void* weight, float alpha,
             float* sigma, void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (!act_absmax || !weight || !sigma)
    return fail(HQ_ERR_INVALID_ARG, "act_absmax, weight and sigma must be non-NULL");
  if (misaligned(act_absmax) || misaligned(weight) || misaligned(sigma))
    return fail(HQ_ERR_INVALID_ARG, "act_absmax, weight and sigma must be 16-byte aligned");
  if (!(alpha >= 0.0f && alpha <= 1.0f))
    return fail(HQ_ERR_INVALID_ARG, "alpha must lie in [0, 1] (got %g)", double(alpha));
  hipStream_t s = static_cast<hipStream_t>(stream);
  // Weight channel maxima land in `sigma`, then are turned into sigma in place.
  hipError_t e = hq::launch_col_absmax(weight, desc->w_dtype == HQ_BF16, desc->d_out, desc->d_in,
                                       sigma, s);
  if (e == hipSuccess) e = hq::launch_sigma_finish(act_absmax, alpha, 1e-5f, desc->d_in, sigma, s);
  return e == hipSuccess ? HQ_OK : hip_fail(e, "sigma kernel launch");
}

int hq_prepare_weights(const hq_desc* desc, const void* weight, const float* bias,
                       const float* sigma, const void* L1, const void* L2, void* prepared,
                       void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (!weight || !prepared) return fail(HQ_ERR_INVALID_ARG, "weight and prepared must be non-NULL");
  if (desc->smooth && !sigma) return fail(HQ_ERR_INVALID_ARG, "smooth = 1 needs sigma");
  if (!desc->smooth && sigma) return fail(HQ_ERR_INVALID_ARG, "smooth = 0 takes no sigma");
  if (desc->rank && (!L1 || !L2)) return fail(HQ_ERR_INVALID_ARG, "rank > 0 needs L1 and L2");
  if (!desc->rank && (L1 || L2)) return fail(HQ_ERR_INVALID_ARG, "rank = 0 takes no L1/L2");
  if (misaligned(weight) || misaligned(prepared) || misaligned(bias) || misaligned(sigma) ||
      misaligned(L1) || misaligned(L2))
    return fail(HQ_ERR_INVALID_ARG,
                "weight, bias, sigma, L1, L2 and prepared must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hq_prepared_layout L;
  layout_of(desc, &L);
  const int64_t np = L.d_out_pad, dout = desc->d_out, din = desc->d_in;
  hipError_t e = hipSuccess;
  // Padding rows of the code matrix and of the per-channel vectors are zero.
  // E2M3 rows past d_out can share a row group with real rows (their bytes
  // interleave slice by slice), so the whole code matrix is cleared first.
  const int fmt = code_fmt_of(desc);
  if (np > dout) {
    const size_t used = fmt == hq::CODES_E2M3 ? 0 : hq::code_bytes(fmt, dout, int(din));
    e = hq::launch_fill_u8(at<uint8_t>(prepared, L.w_codes + used), 0,
                           hq::code_bytes(fmt, np, int(din)) - used, s);
  }
  if (e == hipSuccess)
    e = hq::launch_fill_u32(at<uint32_t>(prepared, L.w_scale), 0u, (L.sigma_inv - L.w_scale) / 4, s);
  if (e == hipSuccess) {
    if (desc->smooth)
      e = hq::launch_reciprocal(sigma, at<float>(prepared, L.sigma_inv), int(din), s);
    else
      e = hq::launch_fill_u32(at<uint32_t>(prepared, L.sigma_inv), 0x3F800000u, size_t(din), s);
  }
  if (e == hipSuccess && bias) e = hq::launch_copy_f32(bias, at<float>(prepared, L.bias), size_t(dout), s);
  if (e == hipSuccess) {
    hq::RowArgs a = {};
    a.in = weight;
    a.in_bf16 = desc->w_dtype == HQ_BF16;
    a.rows = dout;
    a.d = int(din);
    a.scale = desc->smooth ? sigma : nullptr;
    a.log2b = log2i(desc->block);
    a.center = 0;
    a.qmax = qmax_of(desc->w_bits);
    a.codes = at<uint8_t>(prepared, L.w_codes);
    a.code_fmt = fmt;
    a.out_s = at<float>(prepared, L.w_scale);
    a.group = desc->group;
    a.s_ld = np;
    // c = 1^T W~ (the per-token correction); zero under per-channel centring,
    // whose correction is the per-call bias instead.
    a.out_aux = desc->center != HQ_CENTER_CHANNEL ? at<float>(prepared, L.c) : nullptr;
    a.mode = hq::ROW_WEIGHT;
    e = hq::launch_row_transform(a, s);
  }
  if (e == hipSuccess && desc->center == HQ_CENTER_CHANNEL)
    e = hq::launch_copy_f32(static_cast<const float*>(weight), at<float>(prepared, L.weight),
                            size_t(desc->w_dtype == HQ_BF16 ? 2 : 4) * size_t(dout) * din / 4, s);
  if (e == hipSuccess && desc->rank) {
    e = hq::launch_prep_l1(L1, desc->w_dtype == HQ_BF16,
                           desc->smooth ? at<float>(prepared, L.sigma_inv) : nullptr, int(din),
                           desc->rank, at<uint16_t>(prepared, L.l1_hi),
                           at<uint16_t>(prepared, L.l1_lo), s);
    if (e == hipSuccess)
      e = hq::launch_prep_l2(L2, desc->w_dtype == HQ_BF16, desc->rank, int(dout), int(np),
                             at<uint16_t>(prepared, L.l2_hi), at<uint16_t>(prepared, L.l2_lo), s);
  }
  if (e == hipSuccess) {
    PreparedHeader h = {};
    h.magic = kMagic;
    h.version = HQ_ABI_VERSION;
    h.desc = *desc;
    h.d_out_pad = np;
    h.total = L.total;
    e = hq::launch_write_header(&h, sizeof(h), prepared, s);
  }
  return e == hipSuccess ? HQ_OK : hip_fail(e, "prepare kernel launch");
}

int hq_check_prepared(const hq_desc* desc, const void* prepared, void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (!prepared) return fail(HQ_ERR_INVALID_ARG, "prepared is NULL");
  PreparedHeader h;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(&h, prepared, sizeof(h), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "reading the prepared header");
  hq_prepared_layout L;
  layout_of(desc, &L);
  if (h.magic != kMagic) return fail(HQ_ERR_BAD_PREPARED, "prepared blob has no libhq header");
  if (h.version != HQ_ABI_VERSION)
    return fail(HQ_ERR_BAD_PREPARED, "prepared blob version %u != %d", h.version, HQ_ABI_VERSION);
  if (std::memcmp(&h.desc, desc, sizeof(hq_desc)) != 0 || h.total != L.total)
    return fail(HQ_ERR_BAD_PREPARED, "prepared blob was made for a different descriptor");
  return HQ_OK;
}

int hq_quant_linear(const hq_desc* desc, const void* prepared, const void* X, int64_t T, void* Y,
                    void* workspace, size_t workspace_bytes, void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
  if (T == 0) return HQ_OK;
  if (!prepared || !X || !Y || !workspace)
    return fail(HQ_ERR_INVALID_ARG, "prepared, X, Y and workspace must be non-NULL");
  if (misaligned(X) || misaligned(Y) || misaligned(workspace) || misaligned(prepared))
    return fail(HQ_ERR_INVALID_ARG, "X, Y, workspace and prepared must be 16-byte aligned");
  const Workspace w = workspace_of(desc, T);
  if (workspace_bytes < w.total)
    return fail(HQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, w.total);
  hipStream_t s = static_cast<hipStream_t>(stream);
  void* codes = at<uint8_t>(workspace, w.codes);
  float* s_x = at<float>(workspace, w.s_x);
  float* mu = at<float>(workspace, w.mu);
  float* U = desc->rank ? at<float>(workspace, w.U) : nullptr;
  float* lr_part = w.lr_part ? at<float>(workspace, w.lr_part) : nullptr;
  if (desc->center == HQ_CENTER_CHANNEL) {
    float* cmean = at<float>(workspace, w.mean);
    float* bias_eff = at<float>(workspace, w.bias_eff);
    st = run_center(desc, prepared, X, T, at<float>(workspace, w.partial), cmean, bias_eff, s);
    if (st == HQ_OK)
      st = run_act(desc, prepared, X, T, codes, s_x, nullptr, cmean, U, s, lr_part);
    if (st != HQ_OK) return st;
    return run_gemm_dequant(desc, prepared, codes, s_x, bias_eff, U, T, Y, s);
  }
  st = run_act(desc, prepared, X, T, codes, s_x, mu, nullptr, U, s, lr_part);
  if (st != HQ_OK) return st;
  return run_gemm_dequant(desc, prepared, codes, s_x, mu, U, T, Y, s);
}

int hq_channel_center(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                      float* mean, float* bias_eff, void* workspace, size_t workspace_bytes,
                      void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (desc->center != HQ_CENTER_CHANNEL)
    return fail(HQ_ERR_INVALID_ARG, "hq_channel_center needs center = 2 (got %d)", desc->center);
  if (T <= 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 1 (got %lld)", (long long)T);
  if (!prepared || !X || !mean || !bias_eff || !workspace)
    return fail(HQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (misaligned(X) || misaligned(workspace) || misaligned(prepared) || misaligned(mean) ||
      misaligned(bias_eff))
    return fail(HQ_ERR_INVALID_ARG,
                "X, mean, bias_eff, workspace and prepared must be 16-byte aligned");
  const Workspace w = workspace_of(desc, T);
  if (workspace_bytes < w.total)
    return fail(HQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, w.total);
  return run_center(desc, prepared, X, T, at<float>(workspace, w.partial), mean, bias_eff,
                    static_cast<hipStream_t>(stream));
}

int hq_act_quantize(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                    void* codes, float* s_x, float* mu, float* U, void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 0");
  if (T == 0) return HQ_OK;
  if (!prepared || !X || !codes || !s_x || !mu || (desc->rank && !U))
    return fail(HQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (misaligned(X) || misaligned(codes) || misaligned(prepared) || misaligned(s_x) ||
      misaligned(mu) || misaligned(U))
    return fail(HQ_ERR_INVALID_ARG, "X, codes, s_x, mu, U and prepared must be 16-byte aligned");
  const bool chan = desc->center == HQ_CENTER_CHANNEL;
  return run_act(desc, prepared, X, T, codes, s_x, chan ? nullptr : mu, chan ? mu : nullptr, U,
                 static_cast<hipStream_t>(stream));
}

int hq_act_quantize_ws(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                       void* codes, float* s_x, float* mu, float* U, void* workspace,
                       size_t workspace_bytes, void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 0");
  if (T == 0) return HQ_OK;
  if (!prepared || !X || !codes || !s_x || !mu || (desc->rank && !U) || !workspace)
    return fail(HQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (misaligned(X) || misaligned(codes) || misaligned(prepared) || misaligned(s_x) ||
      misaligned(mu) || misaligned(U) || misaligned(workspace))
    return fail(HQ_ERR_INVALID_ARG,
                "X, codes, s_x, mu, U, workspace and prepared must be 16-byte aligned");
  const Workspace w = workspace_of(desc, T);
  if (workspace_bytes < w.total)
    return fail(HQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, w.total);
  float* lr_part = w.lr_part ? at<float>(workspace, w.lr_part) : nullptr;
  const bool chan = desc->center == HQ_CENTER_CHANNEL;
  return run_act(desc, prepared, X, T, codes, s_x, chan ? nullptr : mu, chan ? mu : nullptr, U,
                 static_cast<hipStream_t>(stream), lr_part);
}

int hq_act_transform(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                     float* Xt, float* mu, void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 0");
  if (T == 0) return HQ_OK;
  if (!prepared || !X || !Xt || !mu) return fail(HQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (misaligned(X) || misaligned(Xt) || misaligned(prepared) || misaligned(mu))
    return fail(HQ_ERR_INVALID_ARG, "X, Xt, mu and prepared must be 16-byte aligned");
  hq_prepared_layout L;
  layout_of(desc, &L);
  hq::RowArgs a = {};
  a.in = X;
  a.in_bf16 = desc->x_dtype == HQ_BF16;
  a.rows = T;
  a.d = desc->d_in;
  const bool chan = desc->center == HQ_CENTER_CHANNEL;
  a.scale = (desc->smooth || chan) ? at<float>(prepared, L.sigma_inv) : nullptr;
  a.log2b = log2i(desc->block);
  a.chan_mean = chan ? mu : nullptr;
  a.center = desc->center == HQ_CENTER_TOKEN;
  a.qmax = qmax_of(desc->a_bits);
  a.out_aux = chan ? nullptr : mu;
  a.out_xt = Xt;
  a.mode = hq::ROW_EXPORT;
  hipError_t e = hq::launch_row_transform(a, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HQ_OK : hip_fail(e, "transform kernel launch");
}

int hq_gemm_i32(const hq_desc* desc, const void* a_codes, const void* w_codes, int64_t T,
                int64_t N, int32_t* acc, void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0 || N <= 0 || N % 8) return fail(HQ_ERR_INVALID_ARG, "need T >= 0 and N a positive multiple of 8");
  if (T == 0) return HQ_OK;
  if (!a_codes || !w_codes || !acc) return fail(HQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (misaligned(a_codes) || misaligned(w_codes) || misaligned(acc))
    return fail(HQ_ERR_INVALID_ARG, "a_codes, w_codes and acc must be 16-byte aligned");
  hipError_t e = launch_codes_gemm(desc, a_codes, T, w_codes, N, acc, N, nullptr,
                                   static_cast<hipStream_t>(stream));
  return e == hipSuccess ? HQ_OK : hip_fail(e, "GEMM kernel launch");
}

int hq_gemm_dequant(const hq_desc* desc, const void* prepared, const void* codes,
                    const float* s_x, const float* mu, const float* U, int64_t T, void* Y,
                    void* stream) {
  g_err.clear();
  int st = check_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 0");
  if (T == 0) return HQ_OK;
  if (!prepared || !codes || !s_x || !mu || !Y || (desc->rank && !U))
    return fail(HQ_ERR_INVALID_ARG, "a required pointer is NULL");
  if (misaligned(Y) || misaligned(codes) || misaligned(prepared) || misaligned(s_x) ||
      misaligned(mu) || misaligned(U))
    return fail(HQ_ERR_INVALID_ARG, "Y, codes, s_x, mu, U and prepared must be 16-byte aligned");
  return run_gemm_dequant(desc, prepared, codes, s_x, mu, U, T, Y,
                          static_cast<hipStream_t>(stream));
}

int hq_int_validate(const hq_int_desc* desc) {
  g_err.clear();
  return check_int_desc(desc);
}

size_t hq_int_prepared_bytes(const hq_int_desc* desc) {
  g_err.clear();
  if (check_int_desc(desc) != HQ_OK) return 0;
  hq_int_layout L;
  int_layout_of(desc, &L);
  return L.total;
}

int hq_int_prepared_layout_of(const hq_int_desc* desc, hq_int_layout* out) {
  g_err.clear();
  if (!out) return fail(HQ_ERR_INVALID_ARG, "out is NULL");
  int st = check_int_desc(desc);
  if (st != HQ_OK) return st;
  int_layout_of(desc, out);
  return HQ_OK;
}

size_t hq_int_workspace_bytes(const hq_int_desc* desc, int64_t T) {
  g_err.clear();
  if (check_int_desc(desc) != HQ_OK) return 0;
  if (T < 0) {
    fail(HQ_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
    return 0;
  }
  return align256(4 * size_t(T) * int_acc_width(desc));
}

int hq_int_prepare(const hq_int_desc* desc, const void* weight, const float* bias, float s_x,
                   float s_y, float s_z, float s_u, void* prepared, void* stream) {
  g_err.clear();
  int st = check_int_desc(desc);
  if (st != HQ_OK) return st;
  if (!weight || !prepared) return fail(HQ_ERR_INVALID_ARG, "weight and prepared must be non-NULL");
  if (!(s_x > 0.0f) || !(s_y > 0.0f) || !std::isfinite(s_x) || !std::isfinite(s_y))
    return fail(HQ_ERR_INVALID_ARG, "s_x and s_y must be positive and finite (got %g, %g)",
                double(s_x), double(s_y));
  const bool table = desc->act == HQ_INT_ACT_SILU || desc->act == HQ_INT_ACT_GELU;
  if (table && (!(s_z > 0.0f) || !(s_u > 0.0f) || !std::isfinite(s_z) || !std::isfinite(s_u)))
    return fail(HQ_ERR_INVALID_ARG,
                "SiLU/GELU need s_z and s_u positive and finite (got %g, %g)", double(s_z),
                double(s_u));
  if (misaligned(prepared) || misaligned(weight) || misaligned(bias))
    return fail(HQ_ERR_INVALID_ARG, "weight, bias and prepared must be 16-byte aligned");
  hipStream_t s = static_cast<hipStream_t>(stream);
  hq_int_layout L;
  int_layout_of(desc, &L);
  const int64_t np = L.d_out_pad, dout = desc->d_out, din = desc->d_in;
  const int64_t aw = int_acc_width(desc), xw = int_x_width(desc);
  const bool wh = desc->side == HQ_INT_WH;
  hipError_t e = hipSuccess;
  if (np > aw)
    e = hq::launch_fill_u8(at<uint8_t>(prepared, L.w_codes + size_t(aw) * xw), 0,
                           size_t(np - aw) * xw, s);
  if (e == hipSuccess)
    e = hq::launch_fill_u32(at<uint32_t>(prepared, L.w_scale), 0u, size_t(np), s);
  if (e == hipSuccess) {
    if (wh) {
      // W-bar = H_out [W; 0]: butterflies over the output-channel index
      e = hq::launch_wh_weight(weight, desc->w_dtype == HQ_BF16, int(dout), int(aw), int(din),
                               desc->block, at<float>(prepared, L.wbar), s);
    } else {
      // W-bar = [W 0] H_in: the row transform along the (padded) input
      // channels, exported as float; a padded order first writes [W 0] into
      // W-bar's place and transforms it there (each row is read whole before
      // any of it is written)
      hq::RowArgs a = {};
      a.in = weight;
      a.in_bf16 = desc->w_dtype == HQ_BF16;
      if (xw > din) {
        e = hq::launch_pad_rows(weight, desc->w_dtype == HQ_BF16, dout, int(din), int(xw),
                                at<float>(prepared, L.wbar), s);
        a.in = at<float>(prepared, L.wbar);
        a.in_bf16 = 0;
      }
      a.rows = dout;
      a.d = int(xw);
      a.log2b = log2i(desc->in_block);
      a.qmax = 127.0f;
      a.out_xt = at<float>(prepared, L.wbar);
      a.mode = hq::ROW_EXPORT;
      if (e == hipSuccess) e = hq::launch_row_transform(a, s);
    }
  }
  if (e == hipSuccess) {
    // per-output-channel 8-bit codes of W-bar (no further rotation)
    hq::RowArgs a = {};
    a.in = at<float>(prepared, L.wbar);
    a.in_bf16 = 0;
    a.rows = aw;
    a.d = int(xw);
    a.log2b = 0;
    a.qmax = 127.0f;
    a.codes = at<uint8_t>(prepared, L.w_codes);
    a.code_fmt = hq::CODES_I8;
    a.out_s = at<float>(prepared, L.w_scale);
    a.mode = hq::ROW_WEIGHT;
    e = hq::launch_row_transform(a, s);
  }
  if (e == hipSuccess)
    e = hq::launch_int_constants(bias, int(dout), at<float>(prepared, L.w_scale), int(aw),
                                 int(np), desc->block, desc->post_block, desc->act,
                                 wh ? desc->block : 1, s_x, s_y, table ? s_z : 0.0f,
                                 table ? s_u : 0.0f, at<int32_t>(prepared, L.b_int),
                                 at<int32_t>(prepared, L.mult), at<int32_t>(prepared, L.shift),
                                 at<int8_t>(prepared, L.lut), at<int32_t>(prepared, L.mult_in),
                                 at<int32_t>(prepared, L.shift_in), s);
  if (e == hipSuccess) {
    IntHeader h = {};
    h.magic = kMagicInt;
    h.version = HQ_ABI_VERSION;
    h.desc = *desc;
    h.d_out_pad = np;
    h.total = L.total;
    h.s_x = s_x;
    h.s_y = s_y;
    h.s_z = table ? s_z : 0.0f;
    h.s_u = table ? s_u : 0.0f;
    e = hq::launch_write_header(&h, sizeof(h), prepared, s);
  }
  return e == hipSuccess ? HQ_OK : hip_fail(e, "integer-layer prepare kernel launch");
}

int hq_int_linear(const hq_int_desc* desc, const void* prepared, const int8_t* x_codes,
                  int64_t T, int8_t* y_codes, void* workspace, size_t workspace_bytes,
                  void* stream) {
  g_err.clear();
  int st = check_int_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
  if (T == 0) return HQ_OK;
  if (!prepared || !x_codes || !y_codes || !workspace)
    return fail(HQ_ERR_INVALID_ARG, "prepared, x_codes, y_codes and workspace must be non-NULL");
  if (misaligned(x_codes) || misaligned(y_codes) || misaligned(workspace) || misaligned(prepared))
    return fail(HQ_ERR_INVALID_ARG, "x_codes, y_codes, workspace and prepared must be 16-byte aligned");
  const int aw = int_acc_width(desc), xw = int_x_width(desc), ow = int_out_width(desc);
  const size_t need = align256(4 * size_t(T) * aw);
  if (workspace_bytes < need)
    return fail(HQ_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", workspace_bytes, need);
  hipStream_t s = static_cast<hipStream_t>(stream);
  hq_int_layout L;
  int_layout_of(desc, &L);
  if (desc->d_out % 256 == 0 && aw == desc->d_out && ow == desc->d_out) {
    // whole 256-channel units: GEMM and requantisation in one kernel (the
    // same integers as the two-kernel path below)
    const hipError_t e =
        hq::launch_int_fused(x_codes, T, xw, at<int8_t>(prepared, L.w_codes),
                             desc->d_out, transition_of(desc, prepared), y_codes, s);
    return e == hipSuccess ? HQ_OK : hip_fail(e, "integer-layer kernel launch");
  }
  int32_t* acc = static_cast<int32_t*>(workspace);
  hipError_t e = hq::launch_gemm(x_codes, T, at<int8_t>(prepared, L.w_codes), aw, xw, acc, aw,
                                 nullptr, s);
  if (e != hipSuccess) return hip_fail(e, "GEMM kernel launch");
  return run_int_requant(desc, prepared, acc, T, y_codes, s);
}

int hq_int_requant(const hq_int_desc* desc, const void* prepared, const int32_t* acc, int64_t T,
                   int8_t* y_codes, void* stream) {
  g_err.clear();
  int st = check_int_desc(desc);
  if (st != HQ_OK) return st;
  if (T < 0) return fail(HQ_ERR_INVALID_ARG, "T must be >= 0 (got %lld)", (long long)T);
  if (T == 0) return HQ_OK;
  if (!prepared || !acc || !y_codes)
    return fail(HQ_ERR_INVALID_ARG, "prepared, acc and y_codes must be non-NULL");
  if (misaligned(acc) || misaligned(y_codes) || misaligned(prepared))
    return fail(HQ_ERR_INVALID_ARG, "acc, y_codes and prepared must be 16-byte aligned");
  return run_int_requant(desc, prepared, acc, T, y_codes, static_cast<hipStream_t>(stream));
}

}  // extern "C"
