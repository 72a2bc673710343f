"""CPU oracle for the rotated-and-centred quantised linear layer.

TEST INFRASTRUCTURE ONLY. Nothing in the library's product path may import,
call or execute this module: it is used by ``tests/``, by the entry point's
smoke check and by the benchmark's CPU-baseline leg, and nowhere else. It
shares no code with the HIP path (no kernels, helpers, tables or constants).

It is deliberately plain: float64 NumPy, every step in the order the pages
give it, library matrix products as the only building block. Sources (page
titles; equations as numbered on those pages):

* HadaNorm (pith.science review of "HadaNorm: Diffusion Transformer
  Quantization through Mean-Centered Transformations"), section "What
  carries the argument": Eq. (1), the identity
  XW + b = X~ W~ + b~ with X~ = X diag(1/sigma) H - mu,
  W~ = H^T diag(sigma) W, b~ = b + mu W~, and Eq. (3), the smoothing scale
  sigma_i = max|X_i|^alpha / max|W_i|^(1 - alpha); mu is the per-token mean
  of the scaled-and-rotated activations.
* "Hadamard-Domain Model Quantization for Learned Image Coding" (HaTQ):
  Sec. III-A Eq. (3), the symmetric quantiser; Sec. III-B Eq. (4), integer
  accumulation; Sec. III-C Eq. (7)-(8), the normalised Hadamard transform;
  Sec. IV-B Eq. (13)-(14), double-Hadamard quantisation; Sec. IV-C Eq. (23),
  the constant-basis component; Eq. (18), the accumulator scale s_x s_w;
  supplement Sec. VII-A Eq. (32)-(34), the Sylvester construction; Sec. IV-B
  Eq. (15)-(22) with supplement Eq. (40)-(44), the weight-only Hadamard layer
  and its integer requantisation (section "Weight-only Hadamard layer" below).
* "Data-free 4-bit quantization for diffusion transformers" (blog), section
  "Hadamard rotation: the int4 improvement", steps 2-7 and "How it is applied
  here": block-diagonal Hadamard over contiguous channel blocks, and the
  16-bit low-rank branch fed with the smoothed, un-rotated input.

Layout convention: row vectors. X is [T, d_in] (one token per row), the
weight is passed as ``weight`` [d_out, d_in] (W = weight^T), b is [d_out].

Readings taken where the pages leave a step open:

* mu is one scalar per token (the mean over the d_in transformed channels):
  ``center`` 1 (or True). ``center`` 2 takes the other reading of the same
  equation: mu is one vector over the channels, the mean over the T tokens of
  the call of each transformed channel (HadaNorm Fig. 2 caption, "mu, sigma
  in R^d"; "one added token"), and b~ = b + mu W~ is then a single corrected
  bias for every token. ``center`` 0 (or False) leaves mu = 0.
* sigma uses max(., 1e-5) on both maxima; X_i is input channel i over all
  tokens, W_i is input channel i over all outputs.
* H is the normalised Sylvester matrix in natural order, applied per
  contiguous block of ``block`` channels.
* Activations get one scale per token, weights one scale per output
  channel; codes are symmetric in [-qmax, qmax], qmax = 2^(bits-1) - 1.
* The rounding decision is round(v / s) of HaTQ Eq. (3) as written: the
  quotient of the float64 value and the float64 scale, rounded once, half
  to even. The pages state no precision for it, so the oracle takes the
  equation's own (real) arithmetic as closely as float64 gives it. A float32
  evaluation of the same decision can differ only where v / s lies within
  its float32 error of a half-integer; comparisons attribute every such
  difference to a near-tie.
* A row whose maximum is 0 gets scale 0 and all-zero codes.
* The bias correction uses c = 1^T W~ from the unquantised W~.
* The low-rank branch sees x' = x / sigma (smoothed, not rotated, not
  centred) and contributes (x' L1) L2, L1 [d_in, r], L2 [r, d_out].
* ``group`` = 64 (the data-free int4 blog's recipe, "Hadamard rotation: the
  int4 improvement", step 7 and "How it is applied here"): one scale per row
  and group of 64 consecutive channels instead of one per row, for both
  activations and weights; the integer products are summed per group and
  each group's sum is scaled by s_x[t, g] s_w[j, g]. ``group`` = 0 keeps one
  scale per row.
* Y is rounded once, half-to-even, to the output dtype.

Parity status: every step below is pinned by ``tests/test_oracle.py``
(construction and orthogonality of H, brute force on tiny inputs, the exact
identity with quantisation off, closed forms, a hand-worked example). The
end-to-end quantised output has no value printed on the pages; it is fixed
only through the composition of those pinned steps.
"""
from __future__ import annotations

import numpy as np

EPS = 1e-5
CENTER_NONE, CENTER_TOKEN, CENTER_CHANNEL = 0, 1, 2


# --------------------------------------------------------------------------
# Hadamard matrices and the rotation
# --------------------------------------------------------------------------

def sylvester(m: int) -> np.ndarray:
    """Unnormalised Sylvester matrix of order m (a power of two).

    HaTQ supplement Sec. VII-A Eq. (34): start from [1] and double with
    [[H, H], [H, -H]].
    """
    if m < 1 or (m & (m - 1)):
        raise ValueError(f"Sylvester order must be a power of two, got {m}")
    h = np.ones((1, 1))
    while h.shape[0] < m:
        h = np.block([[h, h], [h, -h]])
    return h


def hadamard(m: int) -> np.ndarray:
    """Normalised Hadamard matrix H = H~ / sqrt(m), so H H^T = I (HaTQ Eq. (7), (32)-(33))."""
    return sylvester(m) / np.sqrt(m)


def rotate(x: np.ndarray, block: int) -> np.ndarray:
    """Rows of x times the block-diagonal H = diag(H_B, ..., H_B).

    Each block of ``block`` contiguous channels is transformed on its own
    (HQ-DM Sec. 2.1; blog step 7). Inside a block every output is the
    normalised signed sum of HaTQ Eq. (8). H_B is symmetric, so x H_B equals
    (H_B x^T)^T.
    """
    x = np.asarray(x, dtype=np.float64)
    t, d = x.shape
    if d % block:
        raise ValueError("block must divide the row length")
    return (x.reshape(t, d // block, block) @ hadamard(block)).reshape(t, d)


# --------------------------------------------------------------------------
# Offline: smoothing scales and the weight transform
# --------------------------------------------------------------------------

def smoothing_scales(x_calib: np.ndarray, weight: np.ndarray, alpha: float,
                     eps: float = EPS) -> np.ndarray:
    """sigma_i = max_t |X_ti|^alpha / max_j |W_ij|^(1 - alpha) (HadaNorm Eq. (3)).

    W = weight^T, so W_i (input channel i over all outputs) is column i of
    ``weight``. Both maxima are clamped below at ``eps``.
    """
    ax = np.abs(np.asarray(x_calib, dtype=np.float64)).max(axis=0)
    aw = np.abs(np.asarray(weight, dtype=np.float64)).max(axis=0)
    return np.maximum(ax, eps) ** alpha / np.maximum(aw, eps) ** (1.0 - alpha)


def transform_weights(weight: np.ndarray, sigma: np.ndarray, block: int):
    """W~ = H^T diag(sigma) W (HadaNorm Eq. (1)), returned row-wise.

    With W = weight^T, W~^T = weight diag(sigma) H, so row j of the result
    is (weight_j * sigma) H. Also returns c = 1^T W~ (c_j = sum_i W~_ij), the
    vector that turns mu into the bias correction mu W~.
    """
    v = np.asarray(weight, dtype=np.float64) * np.asarray(sigma, dtype=np.float64)[None, :]
    wt = rotate(v, block)
    c = wt.sum(axis=1)
    return wt, c


# --------------------------------------------------------------------------
# Online: activation transform, centring, quantisation
# --------------------------------------------------------------------------

def transform_activations(x: np.ndarray, sigma: np.ndarray, block: int, center):
    """X~ = X diag(1/sigma) H - mu (HadaNorm Eq. (1)).

    Returns (x', y, mu, x~) with x' = X / sigma and y = x' H. ``center`` 1 /
    True: mu_t is the mean of row t of y (one value per token) and
    x~ = y - mu[:, None]; ``center`` 2: mu_i is the mean of column i of y
    over the tokens (one value per channel) and x~ = y - mu[None, :];
    ``center`` 0 / False: mu = 0 per token and x~ = y.
    """
    xp = np.asarray(x, dtype=np.float64) / np.asarray(sigma, dtype=np.float64)[None, :]
    y = rotate(xp, block)
    mode = int(center)
    if mode == CENTER_CHANNEL:
        mu = y.mean(axis=0) if y.shape[0] else np.zeros(y.shape[1])
        return xp, y, mu, y - mu[None, :]
    if mode not in (CENTER_NONE, CENTER_TOKEN):
        raise ValueError(f"center must be 0, 1 or 2, got {center}")
    mu = y.mean(axis=1) if mode == CENTER_TOKEN else np.zeros(y.shape[0])
    return xp, y, mu, y - mu[:, None]


def quantize_rows(v: np.ndarray, bits: int):
    """Symmetric per-row quantiser of HaTQ Sec. III-A Eq. (3).

    s = ||v||_inf / qmax with qmax = 2^(bits-1) - 1, and
    q = clamp(round(v / s), -qmax, qmax), round = half to even, all in
    float64. A row whose maximum is 0 gets s = 0 and zero codes.
    Returns (codes int16 [rows, n], s float64 [rows]).
    """
    qmax = 2 ** (bits - 1) - 1
    v = np.asarray(v, dtype=np.float64)
    amax = np.abs(v).max(axis=1) if v.shape[1] else np.zeros(v.shape[0])
    s = amax / qmax
    t = np.zeros_like(v)
    nz = s > 0
    t[nz] = v[nz] / s[nz][:, None]
    q = np.clip(np.rint(t), -qmax, qmax).astype(np.int16)
    return q, s


def quantize_groups(v: np.ndarray, bits: int, group: int):
    """The quantiser of quantize_rows with one scale per row and group of
    ``group`` consecutive channels (blog, "Hadamard rotation: the int4
    improvement": each group of 64 input channels shares one scale): every
    group is quantised on its own. Returns (codes [rows, n], s [rows, n / group])."""
    v = np.asarray(v, dtype=np.float64)
    rows, n = v.shape
    if group <= 0 or n % group:
        raise ValueError("group must divide the row length")
    g = n // group
    q, sc = quantize_rows(v.reshape(rows * g, group), bits)
    return q.reshape(rows, n), sc.reshape(rows, g)


# --------------------------------------------------------------------------
# Integer GEMM, low-rank branch, dequantised output
# --------------------------------------------------------------------------

def int_gemm(qa: np.ndarray, qw: np.ndarray) -> np.ndarray:
    """acc_tj = sum_i qa_ti * qw_ji with zero points 0 (HaTQ Eq. (4)).

    Evaluated as a float64 matrix product of the integer codes: every product
    and every partial sum is an integer of magnitude below 2^53, so the
    product is exact whatever the summation order. Returns int64.
    """
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    if qa.size and qw.size:
        bound = int(np.abs(qa).max()) * int(np.abs(qw).max()) * qa.shape[1]
        assert bound < 2 ** 53
    return (qa.astype(np.float64) @ qw.astype(np.float64).T).astype(np.int64)


def group_product(qa, s_x, qw, s_w, group: int) -> np.ndarray:
    """sum_g s_x[t, g] s_w[j, g] (sum_{k in g} qa_tk qw_jk): the integer product
    of each channel group (exact, int_gemm) scaled by its two group scales."""
    qa = np.asarray(qa)
    qw = np.asarray(qw)
    y = np.zeros((qa.shape[0], qw.shape[0]))
    for g in range(qa.shape[1] // group):
        k = slice(g * group, (g + 1) * group)
        y += int_gemm(qa[:, k], qw[:, k]).astype(np.float64) * (
            np.asarray(s_x, dtype=np.float64)[:, g][:, None]
            * np.asarray(s_w, dtype=np.float64)[:, g][None, :])
    return y


def low_rank(xp: np.ndarray, l1: np.ndarray, l2: np.ndarray):
    """16-bit low-rank branch L2 (L1 x^) in row form (x' L1) L2 (blog steps 3-4, 6).

    x' is the smoothed input before rotation. Returns (U = x' L1, U L2).
    """
    u = np.asarray(xp, dtype=np.float64) @ np.asarray(l1, dtype=np.float64)
    return u, u @ np.asarray(l2, dtype=np.float64)


def dequant_output(acc, s_x, s_w, bias, mu, c, lr=None) -> np.ndarray:
    """Y_tj = s_x,t s_w,j acc_tj + b_j + mu_t c_j (+ low-rank).

    s_x,t s_w,j is the accumulator scale of HaTQ Eq. (18); b + mu W~ is the
    corrected bias of HadaNorm Eq. (1), with mu W~ = mu_t c_j.
    """
    y = (np.asarray(acc, dtype=np.float64) * (np.asarray(s_x, dtype=np.float64)[:, None]
                                              * np.asarray(s_w, dtype=np.float64)[None, :]))
    y = y + np.asarray(bias, dtype=np.float64)[None, :]
    y = y + np.asarray(mu, dtype=np.float64)[:, None] * np.asarray(c, dtype=np.float64)[None, :]
    if lr is not None:
        y = y + lr
    return y


def round_to_dtype(y: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values once, half-to-even, to fp32 or bf16 (returned as float64)."""
    y = np.asarray(y, dtype=np.float64)
    if dtype == "f32":
        return y.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        m, e = np.frexp(y)                      # y = m 2^e, 0.5 <= |m| < 1
        return np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)  # 8 significant bits
    raise ValueError(dtype)


def exact_output(x, weight, bias, xp=None, l1=None, l2=None) -> np.ndarray:
    """The unquantised layer X W + b (+ x' L1 L2) in float64 (reference only)."""
    y = np.asarray(x, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T
    y = y + np.asarray(bias, dtype=np.float64)[None, :]
    if l1 is not None:
        y = y + low_rank(xp, l1, l2)[1]
    return y


# --------------------------------------------------------------------------
# The whole layer
# --------------------------------------------------------------------------

def prepare_weights(weight, sigma, block: int, w_bits: int, group: int = 0):
    """Offline half: W~, c, per-output-channel (or per channel and group) codes and scales."""
    wt, c = transform_weights(weight, sigma, block)
    qw, s_w = quantize_groups(wt, w_bits, group) if group else quantize_rows(wt, w_bits)
    return {"wt": wt, "c": c, "qw": qw, "s_w": s_w, "group": group}


def channel_bias(bias, wt, mu_c) -> np.ndarray:
    """b~ = b + mu W~ for a per-channel mu (HadaNorm Eq. (1), center = 2): W~ = wt^T,
    so mu W~ is wt @ mu, one corrected bias shared by every token."""
    return np.asarray(bias, dtype=np.float64) + np.asarray(wt, dtype=np.float64) @ np.asarray(
        mu_c, dtype=np.float64)


def quant_linear(x, prepared, bias, sigma, *, block: int, a_bits: int, center,
                 l1=None, l2=None, out_dtype: str = "f32"):
    """Online half for the rows of ``x``: transform, centre, quantise, integer GEMM, dequantise."""
    xp, y, mu, xt = transform_activations(x, sigma, block, center)
    group = prepared.get("group", 0)
    if group:
        qa, s_x = quantize_groups(xt, a_bits, group)
        acc = None
        # per-group scaled products; the rest of the epilogue as below with unit scales
        acc_in = group_product(qa, s_x, prepared["qw"], prepared["s_w"], group)
        sx_in, sw_in = np.ones(len(xt)), np.ones(len(prepared["qw"]))
    else:
        qa, s_x = quantize_rows(xt, a_bits)
        acc = acc_in = int_gemm(qa, prepared["qw"])
        sx_in, sw_in = s_x, prepared["s_w"]
    u = lr = None
    if l1 is not None:
        u, lr = low_rank(xp, l1, l2)
    if int(center) == CENTER_CHANNEL:
        bias_eff = channel_bias(bias, prepared["wt"], mu)
        y_full = dequant_output(acc_in, sx_in, sw_in, bias_eff, np.zeros(len(xt)),
                                prepared["c"], lr)
    else:
        bias_eff = np.asarray(bias, dtype=np.float64)
        y_full = dequant_output(acc_in, sx_in, sw_in, bias, mu, prepared["c"], lr)
    return {"xp": xp, "y": y, "mu": mu, "xt": xt, "qa": qa, "s_x": s_x, "acc": acc,
            "u": u, "lr": lr, "bias_eff": bias_eff, "y_full": y_full,
            "y_out": round_to_dtype(y_full, out_dtype)}


def run(x, weight, bias, *, block: int, a_bits: int, w_bits: int, center,
        sigma=None, l1=None, l2=None, out_dtype: str = "f32", group: int = 0):
    """Prepare + quant_linear in one call; sigma defaults to ones."""
    d_in = np.asarray(x).shape[1]
    sigma = np.ones(d_in) if sigma is None else np.asarray(sigma, dtype=np.float64)
    prep = prepare_weights(weight, sigma, block, w_bits, group)
    out = quant_linear(x, prep, bias, sigma, block=block, a_bits=a_bits, center=center,
                       l1=l1, l2=l2, out_dtype=out_dtype)
    out.update(prep)
    out["sigma"] = sigma
    return out


# --------------------------------------------------------------------------
# Diagnostics (not parity gates)
# --------------------------------------------------------------------------
# Integer-only DH and WH layers with integer requantisation
# --------------------------------------------------------------------------
#
# HaTQ Sec. IV-B. A weight-only Hadamard (WH) layer transforms the weight
# along its output channels, W-bar = H_out W (supplement Eq. (40): T_out =
# H_out is symmetric, so (T_out)^T W = H_out W, and b-bar = b H_out); its
# activation stays in the original basis. A double-Hadamard (DH) layer
# transforms the weight along its input channels, W-bar = W H_in (Eq. (13)),
# keeps b-bar = b (supplement Sec. VIII-B), and receives its activation
# already in the H_in basis. Either way the int8 product is moved onto the
# next layer's int8 grid with integers only (Eq. (19)-(22) with the identity
# activation): one unnormalised transform of order m over the output
# channels with gamma = sqrt(m), which for a WH layer followed by a WH layer
# restores the original basis (Table I, WH-to-WH), for a DH layer followed by
# a DH layer produces the next layer's H_in basis (DH-to-DH), and with m = 1
# is no transform (DH-to-WH).
#
# With an activation phi between the layers (Table I, Eq. (20)-(22); supplement
# Sec. VIII-C Eq. (45)-(49)) the transition has two transforms: ``block`` (the
# output-side H_out of a WH layer, before phi) and ``post_block`` (the next
# layer's input-side H_in when that layer is DH, after phi); WH-to-DH uses
# both. For phi = identity or ReLU (positively homogeneous) one multiplier per
# channel and one shift carry the whole transition:
#   y = clamp(round(H~_post(phi(H~_block(M . a))) / 2^n)),
#   rho_c = s_A,c / (sqrt(block post_block) s_y).
# For SiLU and GELU (not homogeneous) the pre-activation goes onto its own int8
# grid s_z first, phi runs as a 255-entry integer lookup table, and a second
# multiplier-shift pair moves the result onto the next layer's grid:
#   z = clamp(round(H~_block(M_out . a) / 2^n_out)),  M_out ~ 2^n_out s_A / (sqrt(block) s_z)
#   u = LUT[z] = clamp(round(phi(s_z z) / s_u))
#   y = clamp(round(H~_post(M_in u) / 2^n_in)),        M_in ~ 2^n_in s_u / (sqrt(post_block) s_y)
# Readings taken where the pages leave a step open:
# * H is the normalised Sylvester matrix of the stated order (a power of two
#   dividing the channel count), block-diagonal over contiguous blocks; the
#   full order is the pages' transform. Padded or Paley orders are not built.
# * M_c = round(2^n rho_c) with one shared shift n: the largest n in [0, 48]
#   for which every M_c fits the multiplier bound, the multiplier-precision
#   and overflow constraints of Eq. (19); n = 0 when every rho_c is 0. The
#   bound is 32767 (a positive 16-bit integer) unless the transforms' growth
#   needs less: with block * post_block = 2^L the bound is
#   min(32767, 2^(24 - L) - 1), so that |H~ H~ (M a)| stays below 2^52
#   (two order-256 transforms: M <= 255).
# * A DH layer has no output-side transform (Table I: H_out = I for DH): with
#   an activation its next-layer transform goes in ``post_block`` and
#   ``block`` must be 1. Without one (phi = identity) the two positions give
#   the same integers.
# * GELU is x Phi(x) with the Gaussian CDF (the erf form), SiLU x / (1 + e^-x);
#   the table is built in float64 and rounded half to even.
# * Padded orders (supplement Sec. VII-B Eq. (35)-(41)), Sylvester orders
#   only: a transform order m larger than the channel count C pads the
#   channels with zeros, T = P_C H_m with P_C = [I_C 0]. A WH layer with
#   ``block`` m > d_out holds W-bar = H_m [W; 0] and b-bar = [b 0] H_m (m
#   accumulator channels) and keeps the first d_out channels after H~_m (the
#   projection P_C); a DH layer with ``in_block`` m > d_in holds W-bar =
#   [W 0] H_m and takes m-channel input codes (the previous layer's padded
#   output); ``post_block`` m > d_out pads the activation's d_out channels
#   with zeros before H~_post, so the output has m channels. Eq. (35) picks
#   the smallest supported m >= 4 ceil(C / 4); any larger power of two
#   gives the same identities and is accepted.
# * Bias codes saturate at +-2^27: with |a| <= 127^2 d_in <= 2^27 and M <= 32767,
#   every intermediate of the requantisation then stays below 2^51 in magnitude.
# * round() is round half to even throughout, on exact rationals.
# * Codes are symmetric in [-qmax, qmax] (qmax = 127 for 8 bits).

RQ_MULT_MAX = 32767
RQ_SHIFT_MAX = 48
RQ_BIAS_MAX = 2 ** 27


def round_half_even_shift(v, n: int) -> np.ndarray:
    """round(v / 2^n), ties to even, for integer v (exact; numpy int64)."""
    v = np.asarray(v, dtype=np.int64)
    if n == 0:
        return v.copy()
    q = v >> n                      # floor division (arithmetic shift)
    r = v - (q << n)                # 0 <= r < 2^n
    half = np.int64(1) << (n - 1)
    up = (r > half) | ((r == half) & ((q & 1) == 1))
    return q + up.astype(np.int64)


def requant_shift(rho, mult_max: int = RQ_MULT_MAX) -> int:
    """The shared right shift n of Eq. (19) (see the reading above)."""
    rho = np.asarray(rho, dtype=np.float64)
    top = float(rho.max()) if rho.size else 0.0
    if top <= 0.0:
        return 0
    n = 0
    while n < RQ_SHIFT_MAX and np.rint(top * 2.0 ** (n + 1)) <= mult_max:
        n += 1
    return n


def mult_bound(orders: int) -> int:
    """Multiplier bound for transforms whose orders multiply to ``orders``:
    |a + b_int| < 2^28, so M < 2^(24 - log2(orders)) keeps every output of the
    unnormalised transforms below 2^52 (see the reading above)."""
    lg = int(orders).bit_length() - 1
    return min(RQ_MULT_MAX, 2 ** (24 - lg) - 1)


ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU = 0, 1, 2, 3


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def gelu(x):
    from scipy.special import erf
    x = np.asarray(x, dtype=np.float64)
    return 0.5 * x * (1.0 + erf(x / np.sqrt(2.0)))


PHI = {ACT_SILU: silu, ACT_GELU: gelu}


def act_table(phi, s_z: float, s_u: float, bits: int = 8) -> np.ndarray:
    """The integer activation of Eq. (47) as a table over the int8 grid:
    entry z + qmax = clamp(round(phi(s_z z) / s_u), +-qmax) for |z| <= qmax."""
    qmax = 2 ** (bits - 1) - 1
    z = np.arange(-qmax, qmax + 1, dtype=np.float64)
    return np.clip(np.rint(phi(float(s_z) * z) / float(s_u)), -qmax, qmax).astype(np.int64)


def unnormalised_transform(u, block: int) -> np.ndarray:
    """The integer transform of Eq. (20): each block of ``block`` channels of
    every row multiplied by the +-1 Sylvester matrix (additions and
    subtractions only; exact in int64)."""
    u = np.asarray(u, dtype=np.int64)
    t, d = u.shape
    h = sylvester(block).astype(np.int64)
    return (u.reshape(t, d // block, block) @ h).reshape(t, d)


SIDE_WH, SIDE_DH = 0, 1


def int_prepare(weight, bias, s_x: float, s_y: float, block: int, side: int = SIDE_WH,
                in_block: int = 1, w_bits: int = 8, act: int = ACT_NONE, post_block: int = 1,
                s_z: float = 0.0, s_u: float = 0.0, phi=None):
    """Offline half of an integer-only layer (HaTQ Eq. (13)-(19), supplement
    Eq. (40)-(49)).

    weight [d_out, d_in] (row c = output channel c), bias [d_out], s_x the
    static scale of the int8 input, s_y the scale of the int8 output (the
    next layer's input scale), block = m, the order of the output-side
    integer transform (for WH also the order of H_out on the weight), side
    SIDE_WH or SIDE_DH, in_block the order of H_in on a DH weight.
    act: ACT_NONE, ACT_RELU, ACT_SILU or ACT_GELU (``phi``, a float64
    function, overrides the SiLU/GELU table's function); post_block: the
    order of the transform after the activation (the next layer's H_in);
    s_z, s_u: the int8 grids before and after a SiLU/GELU table.
    Returns W-bar, b-bar, the weight codes and scales, the bias codes
    b_int = round(b-bar / (s_x s_w)), rho, the shift n and the multipliers M
    (for SiLU/GELU: M_out and n_out, plus the table, M_in and n_in)."""
    weight = np.asarray(weight, dtype=np.float64)
    d_out, d_in = weight.shape

    def order_ok(m, c):
        # a power of two dividing c (block-diagonal) or above it (one padded block)
        return m >= 1 and not (m & (m - 1)) and (c % m == 0 or m > c)
    if not order_ok(block, d_out) or (side == SIDE_DH and block > d_out):
        raise ValueError("block must be a power of two dividing d_out (WH: or above it)")
    if not order_ok(post_block, d_out):
        raise ValueError("post_block must be a power of two dividing d_out or above it")
    if act not in (ACT_NONE, ACT_RELU, ACT_SILU, ACT_GELU):
        raise ValueError(f"unknown activation {act}")
    if side == SIDE_DH and act != ACT_NONE and block != 1:
        raise ValueError("a DH layer has no output-side transform: use post_block")
    general = act in (ACT_SILU, ACT_GELU)
    if general and not (s_z > 0 and s_u > 0):
        raise ValueError("SiLU/GELU need the grids s_z > 0 and s_u > 0")
    bias = np.asarray(bias, dtype=np.float64)
    if side == SIDE_WH:
        # H_out acts on the output-channel index: column-wise on weight, row-wise on b;
        # a padded order first appends zero output channels (Eq. (40) with T_out = P H_m)
        acc = max(block, d_out)
        wpad = np.zeros((acc, d_in))
        wpad[:d_out] = weight
        bpad = np.zeros(acc)
        bpad[:d_out] = bias
        wbar = rotate(wpad.T, block).T
        bbar = rotate(bpad[None, :], block)[0]
    elif side == SIDE_DH:
        if not order_ok(in_block, d_in):
            raise ValueError("in_block must be a power of two dividing d_in or above it")
        # Eq. (39): the input channels padded to in_block, then H_in along them
        wpad = np.zeros((d_out, max(in_block, d_in)))
        wpad[:, :d_in] = weight
        wbar = rotate(wpad, in_block)
        bbar = bias.copy()
    else:
        raise ValueError(f"side must be SIDE_WH or SIDE_DH, got {side}")
    qw, s_w = quantize_rows(wbar, w_bits)
    s_a = float(s_x) * s_w
    b_int = np.zeros(wbar.shape[0], dtype=np.int64)
    nz = s_a > 0
    b_int[nz] = np.clip(np.rint(bbar[nz] / s_a[nz]), -RQ_BIAS_MAX, RQ_BIAS_MAX).astype(np.int64)
    out = {"wbar": wbar, "bbar": bbar, "qw": qw, "s_w": s_w, "b_int": b_int, "block": block,
           "side": side, "in_block": in_block, "s_x": float(s_x), "s_y": float(s_y), "act": act,
           "post_block": post_block, "d_out": d_out}
    if not general:
        # Eq. (19): one multiplier per channel and one shift for the whole
        # transition (ReLU commutes with the common factor 2^-n, Eq. (20)-(22))
        rho = s_a / (np.sqrt(block * post_block) * float(s_y))
        n = requant_shift(rho, mult_bound(block * post_block))
        out.update(rho=rho, shift=n, mult=np.rint(rho * 2.0 ** n).astype(np.int64))
        return out
    # Eq. (45): onto the pre-activation grid s_z, before the output-side transform
    rho = s_a / (np.sqrt(block) * float(s_z))
    n = requant_shift(rho, mult_bound(block))
    # Eq. (47): the integer activation; Eq. (48): onto the next layer's grid
    rho_in = float(s_u) / (np.sqrt(post_block) * float(s_y))
    n_in = requant_shift(np.array([rho_in]))
    out.update(rho=rho, shift=n, mult=np.rint(rho * 2.0 ** n).astype(np.int64),
               lut=act_table(phi or PHI[act], s_z, s_u), rho_in=rho_in, shift_in=n_in,
               mult_in=int(np.rint(rho_in * 2.0 ** n_in)), s_z=float(s_z), s_u=float(s_u))
    return out


def int_forward(x_int, prep, bits: int = 8) -> dict:
    """Online integer path: a = x_int w-bar_int^T + b_int (Eq. (4)),
    v = H~_block (M . a) (Eq. (20); Eq. (46) with M_out),
    then the activation and the transform after it:
    identity / ReLU (Eq. (21)-(22)): y = clamp(round(H~_post(phi(v)) / 2^n));
    SiLU / GELU (Eq. (46)-(49)): z = clamp(round(v / 2^n_out)), u = LUT[z],
    y = clamp(round(H~_post(M_in u) / 2^n_in)).
    x_int is the int8 input in the layer's own basis (the original one for
    WH, the H_in basis for DH)."""
    qmax = 2 ** (bits - 1) - 1
    a = int_gemm(x_int, prep["qw"]) + prep["b_int"][None, :]
    u = a * prep["mult"][None, :]
    v = unnormalised_transform(u, prep["block"])
    d_out = prep.get("d_out", v.shape[1])
    v = v[:, :d_out]   # a padded WH order keeps the first d_out channels (P_C)
    out = {"acc": a, "u": u, "v": v}
    act = prep.get("act", ACT_NONE)
    post = prep.get("post_block", 1)

    def pad(t):
        # a padded post order appends zero channels up to post_block
        if post <= t.shape[1]:
            return t
        return np.concatenate([t, np.zeros((t.shape[0], post - t.shape[1]), t.dtype)], axis=1)
    if act in (ACT_NONE, ACT_RELU):
        pv = np.maximum(v, 0) if act == ACT_RELU else v
        w = unnormalised_transform(pad(pv), post)
        y = np.clip(round_half_even_shift(w, prep["shift"]), -qmax, qmax)
    else:
        z = np.clip(round_half_even_shift(v, prep["shift"]), -qmax, qmax)
        ua = prep["lut"][z + qmax]
        w = unnormalised_transform(pad(ua * prep["mult_in"]), post)
        y = np.clip(round_half_even_shift(w, prep["shift_in"]), -qmax, qmax)
        out.update(z=z, u_act=ua)
    out.update(w=w, y_int=y.astype(np.int16))
    return out


def _relu(v):
    return np.maximum(v, 0.0)


def int_dequant_reference(x_int, prep, phi=None) -> np.ndarray:
    """The dequantised output with the bias codes through the normalised
    transforms and the activation, in units of s_y (float64):
    phi((s_A . a) H_block) H_post / s_y. For WH this is Eq. (17) in the
    original basis; for DH the output of Eq. (14) in the next layer's H_in
    basis. No intermediate grid (s_z, s_u) is applied."""
    act = prep.get("act", ACT_NONE)
    if phi is None:
        phi = {ACT_NONE: (lambda v: v), ACT_RELU: _relu}.get(act) or PHI[act]
    a = int_gemm(x_int, prep["qw"]) + prep["b_int"][None, :]
    ya = a.astype(np.float64) * (prep["s_x"] * prep["s_w"])[None, :]
    v = phi(rotate(ya, prep["block"])[:, :prep.get("d_out", ya.shape[1])])
    post = prep.get("post_block", 1)
    if post > v.shape[1]:
        v = np.concatenate([v, np.zeros((v.shape[0], post - v.shape[1]))], axis=1)
    return rotate(v, post) / prep["s_y"]


def quantize_static(x, s: float, bits: int = 8) -> np.ndarray:
    """Per-tensor symmetric quantisation with a fixed scale (the int8 operand
    of Sec. III-B): clamp(round(x / s), +-qmax), ties to even."""
    qmax = 2 ** (bits - 1) - 1
    return np.clip(np.rint(np.asarray(x, dtype=np.float64) / s), -qmax, qmax).astype(np.int16)


# --------------------------------------------------------------------------

def sqnr_db(ref: np.ndarray, approx: np.ndarray) -> float:
    """10 log10(||X||^2 / ||X - X^||^2) (HaTQ Sec. IV-A Eq. (10))."""
    ref = np.asarray(ref, dtype=np.float64)
    err = ref - np.asarray(approx, dtype=np.float64)
    return float(10.0 * np.log10(np.sum(ref * ref) / np.sum(err * err)))


def excess_kurtosis(v: np.ndarray) -> float:
    """Empirical excess kurtosis of all entries (HaTQ Sec. IV-A Eq. (9))."""
    v = np.asarray(v, dtype=np.float64).ravel()
    d = v - v.mean()
    return float(np.mean(d ** 4) / np.mean(d ** 2) ** 2 - 3.0)
