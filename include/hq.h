/*
 * hq.h -- C ABI of libhq: the rotated-and-centred low-bit linear layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (HadaNorm, "What carries the argument", Eq. (1)):
 *
 *     Y = X W + b  =  X~ W~ + b~,   X~ = X diag(1/sigma) H - mu,
 *                                   W~ = H^T diag(sigma) W,  b~ = b + mu W~
 *
 * X is [T, d_in] (one token per row), W = weight^T with ``weight`` passed as
 * [d_out, d_in] row-major (the nn.Linear layout), H the normalised Sylvester
 * Hadamard matrix applied per contiguous block of ``block`` channels
 * (HaTQ supplement Sec. VII-A Eq. (34); data-free int4 blog, step 7), mu the
 * per-token mean of X diag(1/sigma) H. X~ is quantised per token and W~ per
 * output channel with the symmetric quantiser of HaTQ Sec. III-A Eq. (3)
 * (codes in [-(2^(b-1)-1), 2^(b-1)-1]), multiplied in an integer-exact MFMA
 * GEMM (HaTQ Eq. (4); see "Code formats" below) and dequantised with the
 * accumulator scale s_x s_w (HaTQ Eq. (18)) plus the bias correction:
 *
 *     Y_tj = s_x,t s_w,j acc_tj + b_j + mu_t c_j [+ (x'_t L1) L2_:j],
 *     c = 1^T W~,  x' = x / sigma.
 *
 * The optional rank-r branch (blog steps 3-4) is kept in 16-bit and sees the
 * smoothed, un-rotated input x'.
 *
 * Group-wise scales (hq_desc.group = 64; data-free int4 blog, "Hadamard
 * rotation: the int4 improvement" and "How it is applied here": one scale per
 * group of 64 consecutive input channels). X~ gets one scale per token and
 * group, W~ one per output channel and group, and the accumulator is the sum
 * of the per-group integer products, each scaled by its two group scales:
 *
 *     Y_tj = sum_g s_x[g, t] s_w[g, j] acc_tj^(g) + b_j + mu_t c_j [+ ...],
 *     acc^(g) = the integer product over channels [64 g, 64 g + 64).
 *
 * Scales of G = d_in / 64 groups are stored group-major: s_x as [G, T]
 * (activation stage) and s_w as [G, d_out_pad] (prepared blob).
 *
 * Centring modes (hq_desc.center). HQ_CENTER_TOKEN reads mu as above, one
 * mean per token. HQ_CENTER_CHANNEL takes the other reading of the same
 * identity (HadaNorm Fig. 2 caption: "mu, sigma in R^d"; "one added token"):
 * mu is the mean over the T tokens of one call of each channel of
 * X diag(1/sigma) H, i.e. (mean_t X) diag(1/sigma) H, and the correction
 * mu W~ = (mean_t X) W is a single vector, so
 *
 *     Y_tj = s_x,t s_w,j acc_tj + b~_j,   b~ = b + (mean_t X) W
 *
 * (c is zero in this mode). The mean is taken over the rows of each call, so
 * a token's codes depend on the other tokens of the same call.
 *
 * Conventions for every entry point:
 *  - Pointers are DEVICE pointers unless the comment says (host).
 *  - ``stream`` is a hipStream_t (NULL = the default stream). All GPU work is
 *    enqueued asynchronously on it; no entry point synchronises the host
 *    except where stated.
 *  - The caller allocates and owns every buffer. The library allocates no
 *    device memory and keeps no state besides a thread-local error string.
 *  - Every device array argument (X, Y, weight, bias, sigma, L1, L2,
 *    prepared, workspace, code buffers, scales, means, accumulators) must be
 *    16-byte aligned: the kernels read and write them with 16-byte vector
 *    accesses and direct-to-LDS loads. Checked on the host (any allocator's
 *    base pointer is aligned).
 *  - All arguments are validated on the host before anything is enqueued; on
 *    error nothing is launched, outputs are untouched, a negative hq_status
 *    is returned and hq_last_error() describes the problem. No C++
 *    exception crosses this interface.
 *  - Unsupported combinations are rejected, never coerced.
 *
 * Code formats (hq_code_format). Activation and weight codes of one layer
 * share a format, fixed by the descriptor:
 *  HQ_CODES_I8    (a_bits = 8, w_bits = 8 or gemm = HQ_GEMM_I8): int8,
 *                 row-major [rows, d_in], one byte per code; int32
 *                 accumulation on the int8 MFMA.
 *  HQ_CODES_E2M3  (a_bits = w_bits = 4, gemm = HQ_GEMM_AUTO): each code q in [-7, 7] is stored as
 *                 the 6-bit float E2M3 of the same value (bit 5 sign, bits
 *                 4-3 exponent with bias 1, bits 2-0 mantissa; |q| = 0..7 ->
 *                 0, 8, 16, 20, 24, 26, 28, 30; q = 0 is stored as +0). E2M3
 *                 holds every integer up to 7 exactly, so the FP6 MFMA with
 *                 fp32 accumulation returns the exact integer dot products
 *                 (|acc| <= 49 d_in < 2^24). Rows are grouped by 4: group g
 *                 (rows 4g .. 4g+3) occupies bytes [3 d_in g, 3 d_in (g+1));
 *                 inside it, 128-code slice s of row 4g+i is the 96-byte
 *                 little-endian bit string at byte 384 s + 96 i, code
 *                 128 s + k at bits [6k, 6k+6). A matrix of R rows takes
 *                 hq_code_bytes(desc, R) = ceil(R/4) * 3 d_in bytes; bytes of
 *                 rows past R in the last group are never read as results.
 */
#ifndef HQ_H_
#define HQ_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HQ_ABI_VERSION 8

typedef enum {
  HQ_OK = 0,
  HQ_ERR_INVALID_ARG = -1,   /* null pointer, negative size, bad enum      */
  HQ_ERR_UNSUPPORTED = -2,   /* valid but unsupported shape/option          */
  HQ_ERR_WORKSPACE = -3,     /* workspace smaller than hq_workspace_bytes   */
  HQ_ERR_BAD_PREPARED = -4,  /* prepared blob header does not match desc    */
  HQ_ERR_HIP = -5            /* a HIP runtime call or launch failed         */
} hq_status;

typedef enum { HQ_F32 = 0, HQ_BF16 = 1 } hq_dtype;

typedef enum { HQ_CODES_I8 = 0, HQ_CODES_E2M3 = 1 } hq_code_format_t;

/* GEMM engine: HQ_GEMM_AUTO takes the E2M3 / FP6 MFMA when both code widths
 * are 4 bits and the int8 MFMA otherwise; HQ_GEMM_I8 always uses int8 lanes
 * (int4 codes held losslessly in int8) on the int8 MFMA with int32
 * accumulation. Both return identical accumulators. */
typedef enum { HQ_GEMM_AUTO = 0, HQ_GEMM_I8 = 1 } hq_gemm_engine;

/* Centring of X~ (see "Centring modes" above). */
typedef enum { HQ_CENTER_NONE = 0, HQ_CENTER_TOKEN = 1, HQ_CENTER_CHANNEL = 2 } hq_center_mode;

/* Layer descriptor (plain data, passed by host pointer).
 *  d_in    input channels: a multiple of 128 up to 2048, of 256 up to 4096,
 *          or of 512 up to 8192.
 *  d_out   output channels; multiple of 8, >= 8.
 *  block   Hadamard block size: a power of two dividing d_in (1 = no rotation).
 *  a_bits  activation code width: 4 or 8.
 *  w_bits  weight code width: 4 or 8.
 *  center  hq_center_mode: 1 subtract the per-token mean mu (HadaNorm
 *          centring); 2 subtract the per-channel mean over the call's
 *          tokens; 0 mu = 0.
 *  smooth  1: channel smoothing with the sigma given to hq_prepare_weights;
 *          0: sigma == 1 (no scaling pass over X).
 *  rank    low-rank branch rank: 0 (off) or a multiple of 16 up to 64.
 *  x_dtype dtype of X (hq_dtype).
 *  w_dtype dtype of weight, L1 and L2 (hq_dtype).
 *  y_dtype dtype of Y (hq_dtype).
 *  gemm    GEMM engine (hq_gemm_engine); it also fixes the code format.
 *  group   0: one scale per row; 64: one scale per row and 64-channel group
 *          (needs a_bits = w_bits = 4 and gemm = HQ_GEMM_AUTO).
 * Bias, sigma and every scale are float32. */
typedef struct {
  int32_t d_in, d_out, block, a_bits, w_bits, center, smooth, rank;
  int32_t x_dtype, w_dtype, y_dtype, gemm, group;
} hq_desc;

/* Byte offsets of the arrays inside a prepared blob (all 256-byte aligned). */
typedef struct {
  size_t total;        /* hq_prepared_bytes                                  */
  size_t w_codes;      /* codes of W~^T, d_out_pad rows (row j = out j), in
                          the descriptor's code format                      */
  size_t w_scale;      /* f32   [d_out_pad]        s_w (0 for padding rows);
                          [d_in / 64, d_out_pad] with group = 64           */
  size_t c;            /* f32   [d_out_pad]        c = 1^T W~                   */
  size_t bias;         /* f32   [d_out_pad]        b (0 if none)                */
  size_t sigma_inv;    /* f32   [d_in]             1 / sigma                    */
  size_t l1_hi;        /* bf16  [rank, d_in]       hi part of (diag(1/sigma) L1)^T */
  size_t l1_lo;        /* bf16  [rank, d_in]       lo part (residual)           */
  size_t l2_hi;        /* bf16  [d_out_pad, rank]  hi part of L2^T              */
  size_t l2_lo;        /* bf16  [d_out_pad, rank]  lo part                      */
  size_t weight;       /* w_dtype [d_out, d_in]    copy of weight (center = 2
                          only, for b~ = b + (mean_t X) W; 0 otherwise)     */
  int64_t d_out_pad;   /* d_out rounded up to the GEMM column tile              */
} hq_prepared_layout;

/* Bookkeeping (no step of the method): library ABI version (HQ_ABI_VERSION). */
int hq_abi_version(void);

/* Bookkeeping: text of the last error on the calling thread ("" if none).
 * Never NULL. */
const char* hq_last_error(void);

/* Bookkeeping: static name of a status code. */
const char* hq_status_str(int status);

/* Bookkeeping, host-only: check a descriptor (host pointer). Returns HQ_OK
 * or the error. */
int hq_validate(const hq_desc* desc);

/* Bookkeeping, host-only: size in bytes of the prepared-weight blob for
 * ``desc``; 0 if the descriptor is invalid (see hq_last_error). */
size_t hq_prepared_bytes(const hq_desc* desc);

/* Bookkeeping, host-only: layout of the prepared blob (host pointers). With
 * it a caller reads the arrays of a blob in place (weight codes, s_w, c, b,
 * 1/sigma, the split low-rank factors), so no separate unpacking call exists. */
int hq_prepared_layout_of(const hq_desc* desc, hq_prepared_layout* out);

/* Bookkeeping, host-only: workspace bytes hq_quant_linear needs for T
 * tokens; 0 if invalid. The stage entry points take their buffers as
 * separate arguments, so no view into a workspace is exported. */
size_t hq_workspace_bytes(const hq_desc* desc, int64_t T);

/* Bookkeeping, host-only: the code format of ``desc`` (hq_code_format_t), or
 * a negative hq_status if the descriptor is invalid. */
int hq_code_format(const hq_desc* desc);

/* Bookkeeping, host-only: bytes of a code matrix of ``rows`` rows for
 * ``desc`` (see Code formats); 0 if the descriptor is invalid or rows < 0. */
size_t hq_code_bytes(const hq_desc* desc, int64_t rows);

/* Calibration statistic for the smoothing scale (HadaNorm Eq. (3)):
 * absmax[i] = max_t |X[t, i]| over the T rows of X [T, d_in] (x_dtype).
 * absmax: f32 [d_in], overwritten. T = 0 writes zeros. */
int hq_channel_absmax(const hq_desc* desc, const void* X, int64_t T, float* absmax,
                      void* stream);

/* Smoothing scales, HadaNorm Eq. (3):
 *   sigma_i = max(act_absmax_i, 1e-5)^alpha / max(max_j |weight_ji|, 1e-5)^(1-alpha)
 * act_absmax: f32 [d_in] (from hq_channel_absmax over calibration tokens),
 * weight: [d_out, d_in] (w_dtype), alpha in [0, 1]. sigma: f32 [d_in]. */
int hq_sigma(const hq_desc* desc, const float* act_absmax, const void* weight, float alpha,
             float* sigma, void* stream);

/* Offline weight transform (HadaNorm Eq. (1); HaTQ Sec. IV-D: weight-side
 * transforms are precomputed): for each output row j,
 *   w~_j = (weight_j * sigma) H,  c_j = sum_i w~_ji,
 *   s_w,j = max_i |w~_ji| / qmax,  codes = clamp(round(w~_j / s_w,j), +-qmax)
 *   (with group = 64 the maximum and the scale are taken per 64-channel group),
 * plus 1/sigma, the bias, and for rank > 0 the split low-rank factors.
 *  weight  [d_out, d_in] w_dtype;  bias f32 [d_out] or NULL (zeros);
 *  sigma   f32 [d_in], required iff desc->smooth (sigma > 0);
 *  L1      [d_in, rank] w_dtype, L2 [rank, d_out] w_dtype (both NULL iff rank 0).
 *  prepared  device buffer of hq_prepared_bytes(desc) bytes, fully written.
 * The blob is immutable afterwards and may be shared by concurrent calls. */
int hq_prepare_weights(const hq_desc* desc, const void* weight, const float* bias,
                       const float* sigma, const void* L1, const void* L2, void* prepared,
                       void* stream);

/* Bookkeeping: host-synchronising check that ``prepared`` was written by
 * hq_prepare_weights for this descriptor (reads its 256-byte header). */
int hq_check_prepared(const hq_desc* desc, const void* prepared, void* stream);

/* The hot path: Y = quantised layer(X) for T tokens, i.e. X~ W~ + b~ of
 * HadaNorm Eq. (1) ("What carries the argument") with X~ quantised per token
 * by HaTQ Sec. III-A Eq. (3), the integer product of HaTQ Sec. III-B Eq. (4),
 * the accumulator scale s_x s_w of HaTQ Eq. (18), the bias correction mu W~,
 * and (rank > 0) the 16-bit branch of the data-free int4 blog ("Hadamard
 * rotation: the int4 improvement", steps 3-4).
 *  X [T, d_in] x_dtype, row-major;  Y [T, d_out] y_dtype, row-major.
 *  workspace: device buffer of at least hq_workspace_bytes(desc, T) bytes,
 *  not shared with a concurrent call. T = 0 is a no-op. */
int hq_quant_linear(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                    void* Y, void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the static scratch array of hq_quant_linear_noalloc (per GPU). */
#define HQ_NOALLOC_SCRATCH_BYTES (32u << 20)

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, hosts that forbid allocation): the same
 * computation and kernels as hq_quant_linear, with the workspace in a static
 * device array of HQ_NOALLOC_SCRATCH_BYTES bytes that the library holds on
 * each GPU it runs on until the process ends (its address is looked up on the
 * first call on each device, with that device current). No allocation of any
 * kind happens in the call. Returns HQ_ERR_WORKSPACE, launching nothing, when
 * hq_workspace_bytes(desc, T) exceeds the array. Every call on one GPU shares
 * that GPU's array, so calls that overlap on a GPU (other streams, other host
 * threads) race: the caller serialises them. The array keeps the last call's
 * contents; nothing in it needs clearing (every byte read is first written by
 * the same call). Arguments and errors otherwise as hq_quant_linear;
 * ``stream`` must belong to the current device. */
int hq_quant_linear_noalloc(const hq_desc* desc, const void* prepared, const void* X,
                            int64_t T, void* Y, void* stream);

/* ---- Stage entry points (the same kernels, for testing and profiling) ---- */

/* Per-channel centring statistics (center = 2 only; T >= 1), the per-channel
 * reading of mu in HadaNorm Eq. (1) (Fig. 2 caption: mu in R^d; "one added
 * token"): over the T rows
 * of X, mean f32 [d_in] = mean_t X (the activation stage subtracts it from
 * every token before the channel scaling and the rotation, which yields the
 * same X~ as subtracting mu after them) and bias_eff f32 [d_out_pad] =
 * b + (mean_t X) W (the corrected bias; padding entries 0). Both are summed in
 * a fixed order. workspace: at least hq_workspace_bytes(desc, T) bytes. */
int hq_channel_center(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                      float* mean, float* bias_eff, void* workspace, size_t workspace_bytes,
                      void* stream);

/* Activation stage alone: X~ = X diag(1/sigma) H - mu of HadaNorm Eq. (1),
 * quantised per token (or per token and 64-channel group) by HaTQ Sec. III-A
 * Eq. (3), plus U = x' L1 of the blog's step 3. Outputs: codes of T rows in
 * the descriptor's code format
 * (hq_code_bytes(desc, T) bytes, natural channel order), s_x f32 [T]
 * (dequant scale of the normalised X~ row; [d_in / 64, T] with group = 64,
 * one per token and group), mu f32 [T], U f32 [T, rank]
 * (x' L1; ignored/NULL when rank = 0). For center = 2, mu is instead an
 * INPUT: the mean [d_in] of hq_channel_center. */
int hq_act_quantize(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                    void* codes, float* s_x, float* mu, float* U, void* stream);

/* The activation stage exactly as hq_quant_linear runs it (HadaNorm Eq. (1),
 * HaTQ Sec. III-A Eq. (3), blog steps 3-4): the same outputs as
 * hq_act_quantize, bit for bit, but for rank > 0 the down projection U = x' L1
 * takes the two-pass form that keeps its per-slice products in the workspace
 * (hq_act_quantize, which has no workspace, makes one pass with every block
 * reading all of L1). Where the row transform and the projection run as one
 * launch (bf16 X, d_in 2560 or 3072, block >= 512, rank 16 or 32, center
 * 0 or 1, no groups) both entry points run that launch and the workspace is
 * not written. workspace: at least hq_workspace_bytes(desc, T) bytes (only
 * its slice-product region is written); caller-owned, contents undefined on
 * entry and exit. Returns HQ_ERR_WORKSPACE if too small. */
int hq_act_quantize_ws(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                       void* codes, float* s_x, float* mu, float* U, void* workspace,
                       size_t workspace_bytes, void* stream);

/* Debug export of the float transform before quantisation, X~ of HadaNorm
 * Eq. (1) (H normalised as in HaTQ Eq. (7)):
 * Xt f32 [T, d_in] = X~ (centred if desc->center), mu f32 [T].
 * For center = 2, mu is an INPUT: the mean [d_in] of hq_channel_center. */
int hq_act_transform(const hq_desc* desc, const void* prepared, const void* X, int64_t T,
                     float* Xt, float* mu, void* stream);

/* Integer GEMM alone, HaTQ Sec. III-B Eq. (4) with zero points 0:
 * acc int32 [T, N] = a_codes [T, d_in] . w_codes [N, d_in]^T,
 * both in the descriptor's code format (T and N rows); N a multiple of 8.
 * With group = 64 this is still the product over all d_in channels (the sum
 * of the unscaled per-group products). */
int hq_gemm_i32(const hq_desc* desc, const void* a_codes, const void* w_codes, int64_t T,
                int64_t N, int32_t* acc, void* stream);

/* GEMM + dequant epilogue alone (HaTQ Eq. (4) and the accumulator scale of
 * Eq. (18); the bias correction b + mu W~ of HadaNorm Eq. (1); the blog's
 * low-rank step 4), from activation-stage outputs (layouts as in
 * hq_act_quantize; U NULL when rank = 0). Y [T, d_out] y_dtype. For
 * center = 2, mu is the bias_eff [d_out_pad] of hq_channel_center. */
int hq_gemm_dequant(const hq_desc* desc, const void* prepared, const void* codes,
                    const float* s_x, const float* mu, const float* U, int64_t T, void* Y,
                    void* stream);

/* ---- Integer-only layers: double-Hadamard (DH) and weight-only Hadamard (WH) ----
 *
 * "Hadamard-Domain Model Quantization for Learned Image Coding" (HaTQ),
 * Sec. IV-B Eq. (13)-(17) and supplement Eq. (40): a WH layer transforms its
 * weight along the OUTPUT channels, W-bar = H_out W, and the bias with it,
 * b-bar = b H_out, and takes its int8 activation in the original basis; a DH
 * layer transforms its weight along the INPUT channels, W-bar = W H_in,
 * keeps b-bar = b, and takes its int8 activation already in the H_in basis.
 * The activation has one static per-tensor scale s_x. Integer-only inference
 * (Sec. III-B Eq. (4)-(6), Eq. (18)-(22), supplement Eq. (44)) with the
 * identity activation:
 *
 *     a   = x_int . w-bar_int^T + b_int,   b_int = round(b-bar / (s_x s_w))
 *     y   = clamp(round(H~_m (M . a) / 2^n), -127, 127)
 *     M_c = round(2^n rho_c),  rho_c = s_x s_w,c / (sqrt(m) s_y)
 *
 * With an activation phi between this layer and the next (Table I; Eq. (20)-
 * (22); supplement Sec. VIII-C Eq. (45)-(49)), the transition runs H~_m
 * before phi and H~_p after it (p = post_block: the next layer's H_in order
 * when that layer is DH; WH-to-DH uses both). ReLU is positively homogeneous,
 * so one multiplier per channel and one shift carry the whole transition:
 *
 *     y   = clamp(round(H~_p (relu(H~_m (M . a))) / 2^n), -127, 127)
 *     rho_c = s_x s_w,c / (sqrt(m p) s_y)        (also for phi = identity)
 *
 * SiLU and GELU go through their own int8 grids s_z (before phi) and s_u
 * (after it), phi realised as a 255-entry integer table:
 *
 *     z   = clamp(round(H~_m (M_out . a) / 2^n_out)),  M_out,c ~ 2^n_out s_x s_w,c / (sqrt(m) s_z)
 *     u   = LUT[z] = clamp(round(phi(s_z z) / s_u))
 *     y   = clamp(round(H~_p (M_in u) / 2^n_in)),     M_in ~ 2^n_in s_u / (sqrt(p) s_y)
 *
 * (GELU: x Phi(x) with the Gaussian CDF; SiLU: x / (1 + e^-x).) A DH layer
 * has no output-side transform of its own, so with an activation its m must
 * be 1 and the next layer's H_in goes in p; with phi = identity the two
 * positions give the same integers.
 *
 * Padded orders (supplement Sec. VII-B Eq. (35)-(41); Sylvester orders only):
 * an order above the channel count pads those channels with zeros, T = P H
 * with P = [I 0]. A WH layer with block m > d_out holds W-bar = H_m [W; 0]
 * and b-bar = [b 0] H_m (m accumulator channels) and keeps the first d_out
 * channels after H~_m; a DH layer with in_block > d_in holds W-bar =
 * [W 0] H_in and takes in_block input codes per token (the previous layer's
 * padded output); post_block p > d_out pads the activation's d_out channels
 * to p before H~_p, so the layer writes p output codes per token. Widths:
 * input codes x_w = in_block if DH and in_block > d_in, else d_in;
 * accumulators a_w = block if WH and block > d_out, else d_out; output codes
 * o_w = post_block if post_block > d_out, else d_out.
 *
 * H~_m: the +-1 Sylvester matrix of order m, block-diagonal over d_out / m
 * blocks of output channels (additions and subtractions only). It is Table
 * I's output-side conversion: for a WH layer followed by a WH layer it
 * restores the original basis (m = the layer's H_out order); for a DH layer
 * followed by a DH layer it produces the next layer's H_in basis (m = that
 * layer's H_in order); m = 1 is no transform (DH followed by WH). H (H_in,
 * H_out) is the normalised Sylvester matrix over contiguous blocks. s_w,c:
 * per-output-channel scale of W-bar (8-bit symmetric codes); s_y: the scale
 * of the output codes (the next layer's input scale). n: the largest shift
 * <= 48 with every M_c within the multiplier bound, min(32767, 2^(24 - L) - 1)
 * for transforms whose orders multiply to 2^L (32767 for one transform of
 * order <= 256; 255 for two of order 256). round() is round half to even;
 * bias codes saturate at +-2^27, so every intermediate stays below 2^52 in
 * magnitude. Every online step is exact integer arithmetic (int32 products;
 * after M the kernel carries the integers in float64 registers, exact in
 * that range).
 */
typedef enum { HQ_INT_WH = 0, HQ_INT_DH = 1 } hq_int_side;
typedef enum {
  HQ_INT_ACT_NONE = 0,  /* identity                                   */
  HQ_INT_ACT_RELU = 1,  /* max(x, 0), on the common scale             */
  HQ_INT_ACT_SILU = 2,  /* x / (1 + e^-x), integer table on s_z, s_u  */
  HQ_INT_ACT_GELU = 3   /* x Phi(x), integer table on s_z, s_u        */
} hq_int_act;

typedef struct {
  int32_t d_in;     /* input channels of the weight; the input width x_w follows
                       hq_desc.d_in's rule                                        */
  int32_t d_out;    /* output channels: multiple of 8                             */
  int32_t block;    /* m: output-side transform order, power of two <= 256
                       dividing d_out (for WH also the order of H_out, which may
                       exceed d_out: a padded order)                              */
  int32_t w_dtype;  /* hq_dtype of weight                                         */
  int32_t side;     /* hq_int_side                                                */
  int32_t in_block; /* DH: order of H_in, a power of two dividing d_in or above it
                       (padded); WH: 1                                            */
  int32_t act;      /* hq_int_act between this layer and the next                 */
  int32_t post_block; /* p: transform after the activation (the next layer's H_in
                       order), power of two <= 256 dividing d_out or above it
                       (padded); 1 = none                                         */
} hq_int_desc;

/* Byte offsets of the arrays in an integer-layer prepared blob (256-byte aligned). */
typedef struct {
  size_t total;
  size_t w_codes;   /* int8  [d_out_pad, x_w]   codes of W-bar (padding rows 0)  */
  size_t w_scale;   /* f32   [d_out_pad]        s_w                             */
  size_t b_int;     /* int32 [d_out_pad]        bias codes                      */
  size_t mult;      /* int32 [d_out_pad]        multipliers M                   */
  size_t shift;     /* int32 [1]                shared shift n                  */
  size_t wbar;      /* f32   [a_w, x_w]         W-bar (written by the prepare)  */
  int64_t d_out_pad; /* a_w rounded up to the GEMM tile                         */
  size_t lut;       /* int8  [256]              SiLU/GELU table, entry z + 127  */
  size_t mult_in;   /* int32 [1]                M_in (SiLU/GELU)                */
  size_t shift_in;  /* int32 [1]                n_in (SiLU/GELU)                */
} hq_int_layout;

/* Bookkeeping, host-only: validation, blob size and layout, workspace of
 * hq_int_linear (int32 products [T, a_w]). */
int hq_int_validate(const hq_int_desc* desc);
size_t hq_int_prepared_bytes(const hq_int_desc* desc);
int hq_int_prepared_layout_of(const hq_int_desc* desc, hq_int_layout* out);
size_t hq_int_workspace_bytes(const hq_int_desc* desc, int64_t T);

/* Offline half of an integer-only layer (HaTQ Sec. IV-B Eq. (13)-(19),
 * supplement Eq. (40)-(49)): weight [d_out, d_in] (w_dtype) and bias f32
 * [d_out] (or NULL) into
 * the blob (hq_int_prepared_bytes): W-bar, its int8 codes and scales, the bias
 * codes, the multipliers and the shift (SiLU/GELU: also the table, M_in and
 * n_in). s_x > 0 is the scale of the int8 input, s_y > 0 that of the int8
 * output; s_z, s_u > 0 are the grids around a SiLU/GELU table (ignored for
 * the other activations). */
int hq_int_prepare(const hq_int_desc* desc, const void* weight, const float* bias, float s_x,
                   float s_y, float s_z, float s_u, void* prepared, void* stream);

/* The integer-only hot path (HaTQ Eq. (4), then the requantisation of
 * Eq. (19)-(22), or of supplement Eq. (45)-(49) for SiLU/GELU): y_codes int8
 * [T, o_w] from x_codes int8 [T, x_w] (codes in
 * [-127, 127], row-major, in the layer's input basis): the int8 MFMA product
 * into the workspace, then hq_int_requant's kernel. T = 0 is a no-op. */
int hq_int_linear(const hq_int_desc* desc, const void* prepared, const int8_t* x_codes,
                  int64_t T, int8_t* y_codes, void* workspace, size_t workspace_bytes,
                  void* stream);

/* Requantisation alone (HaTQ Eq. (19)-(22); supplement Eq. (45)-(49)):
 * y_codes int8 [T, o_w] from the int32 products
 * acc [T, a_w] (x_int . w-bar_int^T, WITHOUT the bias codes, which this
 * stage adds). |acc| <= 2^27 (as every product of int8 codes over d_in <= 8192
 * is); larger values are outside the exact range of the kernel. */
int hq_int_requant(const hq_int_desc* desc, const void* prepared, const int32_t* acc, int64_t T,
                   int8_t* y_codes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HQ_H_ */
