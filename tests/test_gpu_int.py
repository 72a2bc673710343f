"""GPU parity of the integer-only layers with integer requantisation: the
weight-only Hadamard (WH) layer and the double-Hadamard (DH) layer (HaTQ
Sec. IV-B Eq. (13)-(22), supplement Eq. (40)-(49)) against the CPU oracle,
with the identity, ReLU, SiLU or GELU activation between a layer and the next
(Table I; the next layer's H_in after the activation).

The online path is integer arithmetic, so it is held to bit-exactness: the
GPU's output codes must equal the oracle's integer path run on the same
constants (read back from the GPU's prepared blob). The offline constants are
decided in float32 (W-bar, s_w) and float64 (the rest) on the GPU and in
float64 by the oracle, so they are compared to the oracle's own constants
with rounding-aware tolerances: W-bar per row to 2e-6, codes equal except
near-ties (tests/parity.py), multipliers and bias codes equal except where the
oracle's value lies within the float32 uncertainty of a half-integer, the
shift equal; SiLU/GELU tables entry for entry except at float64 half-integer
ties. Cases: the lic_wh workload (12288 x 256 -> 256, H_256) as a WH
layer and as a DH layer (DH-to-DH and DH-to-WH) on its first 300 tokens and
at full size; ragged token counts and widths; blocks 1 to 256; bf16 weights;
zero rows; saturated outputs. A DH layer's input is the workload's X in the
layer's H_in basis (the previous DH layer's output).
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_bit_amd as hq
from hadamard_rotated_bit_amd import workloads as WL
from oracle import hq_oracle as O
from parity import check_codes, tdev, to_np

pytestmark = pytest.mark.gpu
DT = {"f32": hq.F32, "bf16": hq.BF16}


ACT_NAME = {hq.HQ_INT_ACT_NONE: "identity", hq.HQ_INT_ACT_RELU: "ReLU",
            hq.HQ_INT_ACT_SILU: "SiLU", hq.HQ_INT_ACT_GELU: "GELU"}
PHI = {hq.HQ_INT_ACT_NONE: lambda v: v, hq.HQ_INT_ACT_RELU: lambda v: np.maximum(v, 0.0),
       hq.HQ_INT_ACT_SILU: O.silu, hq.HQ_INT_ACT_GELU: O.gelu}


class IntCase:
    def __init__(self, w: WL.Workload, T: int, m: int, x=None, s_y_factor: float = 1.0,
                 side: int = hq.HQ_INT_WH, in_block: int = 1, act: int = hq.HQ_INT_ACT_NONE,
                 post: int = 1):
        kind = "WH" if side == hq.HQ_INT_WH else f"DH H_in={in_block}"
        print(f"\n[case] {kind} {w.name} T={T} {w.d_in}->{w.d_out} m={m} {ACT_NAME[act]} "
              f"post={post} {w.dtype}", flush=True)
        self.w, self.T, self.m, self.act, self.post = w, T, m, act, post
        self.x = WL.gen_x(w, T=T) if x is None else x
        self.weight = WL.gen_weight(w)
        self.bias = WL.gen_bias(w)
        # the layer's input in its own basis (H_in for DH), and the float
        # output in the basis the int8 output codes stand for: the activation
        # of the layer's output (in the original basis; a DH layer without an
        # activation may put the next layer's H_in in m), then H_post
        # (padded orders: a DH input of in_block > d_in channels is [X 0] H_in,
        # and a post order above d_out pads the activation with zeros)
        self.desc = hq.IntDesc(w.d_in, w.d_out, m, DT[w.dtype], side, in_block, act, post)
        xw = self.desc.x_width
        self.x_in = self.x if side == hq.HQ_INT_WH else O.rotate(_pad_cols(self.x, xw), in_block)
        y = np.asarray(self.x, dtype=np.float64) @ np.asarray(self.weight, dtype=np.float64).T + \
            self.bias
        y_pre = y if side == hq.HQ_INT_WH else O.rotate(y, m)
        self.y_ref = O.rotate(_pad_cols(PHI[act](y_pre), self.desc.out_width), post)
        self.s_x = float(np.float32(np.abs(self.x_in).max() / 127.0)) if T else 1.0
        s_y = np.abs(self.y_ref).max() / 127.0 if T else 1.0
        self.s_y = float(np.float32(s_y * s_y_factor))
        table = act in (hq.HQ_INT_ACT_SILU, hq.HQ_INT_ACT_GELU)
        self.s_z = float(np.float32(np.abs(y_pre).max() / 127.0)) if table and T else 0.0
        self.s_u = float(np.float32(np.abs(PHI[act](y_pre)).max() / 127.0)) if table and T else 0.0
        if table and not T:
            self.s_z = self.s_u = 1.0
        self.xi = O.quantize_static(self.x_in, self.s_x)
        self.ora = O.int_prepare(self.weight, self.bias, self.s_x, self.s_y, m, side=side,
                                 in_block=in_block, act=act, post_block=post, s_z=self.s_z,
                                 s_u=self.s_u)
        self.prep = hq.int_prepare(self.desc, tdev(self.weight, w.dtype),
                                   torch.from_numpy(self.bias).cuda(), self.s_x, self.s_y,
                                   self.s_z, self.s_u)
        self.X = torch.from_numpy(self.xi.astype(np.int8)).cuda()

    def gpu_constants(self):
        v = hq.int_views(self.desc, self.prep)
        return {"qw": to_np(v["w_codes"]).astype(np.int64), "b_int": to_np(v["b_int"]).astype(np.int64),
                "mult": to_np(v["mult"]).astype(np.int64), "shift": int(to_np(v["shift"])[0]),
                "block": self.m, "s_w": to_np(v["s_w"]).astype(np.float64),
                "wbar": to_np(v["wbar"]).astype(np.float64), "act": self.act,
                "post_block": self.post, "lut": to_np(v["lut"]).astype(np.int64),
                "mult_in": int(to_np(v["mult_in"])[0]), "shift_in": int(to_np(v["shift_in"])[0]),
                "d_out": self.w.d_out}


def _pad_cols(a, width):
    """a with zero columns appended up to `width` (a padded order's P^T)."""
    a = np.asarray(a, dtype=np.float64)
    if a.shape[1] >= width:
        return a
    return np.concatenate([a, np.zeros((a.shape[0], width - a.shape[1]))], axis=1)


def _half_integer_ties(t, d, rel=4e-6):
    """Every nonzero entry of d (GPU minus oracle, at most 1 apart) sits where
    the oracle's unrounded value t is within float32 uncertainty of a half-integer."""
    assert np.abs(d).max() <= 1
    if d.any():
        tt = t[d != 0]
        win = rel * np.abs(tt) + 1e-9
        assert np.all(np.abs(np.abs(tt - np.floor(tt)) - 0.5) <= win)


def check_constants(c: IntCase):
    o, g = c.ora, c.gpu_constants()
    rows = np.linalg.norm(g["wbar"] - o["wbar"], axis=1) / np.maximum(
        np.linalg.norm(o["wbar"], axis=1), 1e-300)
    assert rows.max() <= 2e-6, rows.max()
    np.testing.assert_allclose(g["s_w"], o["s_w"], rtol=2e-6, atol=1e-30)
    ratio = np.divide(o["wbar"], o["s_w"][:, None], out=np.zeros_like(o["wbar"]),
                      where=o["s_w"][:, None] > 0)
    check_codes(g["qw"], o["qw"], ratio, "W-bar codes")
    assert g["shift"] == o["shift"]
    # multipliers: round(2^n rho) with rho from the float32 s_w
    _half_integer_ties(o["rho"] * 2.0 ** o["shift"], g["mult"] - o["mult"])
    # bias codes: round(b-bar / s_A)
    s_a = c.s_x * o["s_w"]
    tb = np.divide(o["bbar"], s_a, out=np.zeros_like(s_a), where=s_a > 0)
    _half_integer_ties(tb, g["b_int"] - o["b_int"])
    if c.act in (hq.HQ_INT_ACT_SILU, hq.HQ_INT_ACT_GELU):
        # the table: clamp(round(phi(s_z z) / s_u)), float64 on both sides
        z = np.arange(-127, 128, dtype=np.float64)
        tl = np.clip(PHI[c.act](c.s_z * z) / c.s_u, -127.4, 127.4)
        _half_integer_ties(tl, g["lut"][:255] - o["lut"], rel=1e-12)
        assert g["lut"][255] == 0
        assert g["shift_in"] == o["shift_in"]
        _half_integer_ties(np.array([o["rho_in"] * 2.0 ** o["shift_in"]]),
                           np.array([g["mult_in"] - o["mult_in"]]), rel=1e-12)
    return g


def check_outputs(c: IntCase, Y):
    g = c.gpu_constants()
    y = to_np(Y).astype(np.int64)
    # bit-exact against the oracle's integer path on the GPU's constants
    ref = O.int_forward(c.xi, g)["y_int"].astype(np.int64)
    assert np.array_equal(y, ref), np.argwhere(y != ref)[:5]
    # and against the oracle's own constants (which differ from the GPU's only
    # in multipliers or bias codes at half-integer ties): nearly everywhere equal
    own = O.int_forward(c.xi, c.ora)["y_int"].astype(np.int64)
    diff = np.abs(y - own)
    if diff.size:
        if c.act == hq.HQ_INT_ACT_NONE and c.post == 1:
            assert diff.max() <= 1
            assert (diff > 0).mean() <= 1e-3, (diff > 0).mean()
        else:
            # a multiplier one apart moves a pre-activation grid point, which
            # the table and H_post can spread over a block
            assert (diff > 0).mean() <= 1e-2, (diff > 0).mean()
            own_sq = O.sqnr_db(c.y_ref / c.s_y, own.astype(np.float64))
            assert abs(O.sqnr_db(c.y_ref / c.s_y, y.astype(np.float64)) - own_sq) < 0.1
    return y


def test_wh_lic_first_rows():
    c = IntCase(WL.WORKLOADS["lic_wh"], 300, 256)
    check_constants(c)
    Y = hq.int_linear(c.desc, c.prep, c.X)
    y = check_outputs(c, Y)
    exact = c.y_ref / c.s_y
    sq = O.sqnr_db(exact, y.astype(np.float64))
    own = O.sqnr_db(exact, O.int_forward(c.xi, c.ora)["y_int"].astype(np.float64))
    print(f"lic_wh: output SQNR {sq:.2f} dB against the float layer (oracle {own:.2f} dB)")
    # the activation keeps its original basis and one per-tensor scale, so the
    # x30 outlier channels coarsen its grid; int8 still reaches ~20 dB here
    assert abs(sq - own) < 0.05 and sq > 15


def test_wh_requant_stage_bit_exact():
    # the requantisation alone on wide int32 products (beyond what 8-bit codes
    # produce), against the oracle's integer steps on the GPU's constants
    c = IntCase(WL.WORKLOADS["lic_wh"], 4, 256)
    g = c.gpu_constants()
    rng = np.random.default_rng(21)
    acc = rng.integers(-2 ** 27, 2 ** 27, (257, c.w.d_out), dtype=np.int64)
    acc[:3] = 0
    acc[3] = 2 ** 27 - 1
    y = to_np(hq.int_requant(c.desc, c.prep, torch.from_numpy(acc.astype(np.int32)).cuda()))
    u = (acc + g["b_int"][None, :]) * g["mult"][None, :]
    v = O.unnormalised_transform(u, c.m)
    ref = np.clip(O.round_half_even_shift(v, g["shift"]), -127, 127)
    assert np.array_equal(y.astype(np.int64), ref)


@pytest.mark.parametrize("T,d_in,d_out,m,dtype", [
    (1, 128, 128, 128, "f32"),
    (3, 384, 136, 8, "f32"),
    (77, 256, 264, 1, "f32"),      # no output transform (gamma = 1)
    (130, 1152, 512, 64, "bf16"),
    (257, 256, 1024, 256, "f32"),  # several 256-channel chunks per row
])
def test_wh_ragged(T, d_in, d_out, m, dtype):
    w = WL.custom(500 + T, T, d_in, d_out, dtype=dtype, x_dist="laplace", n_outliers=3,
                  outlier=20.0, w_std=0.05)
    c = IntCase(w, T, m)
    check_constants(c)
    check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))


def test_wh_zero_rows_pass_the_bias():
    w = WL.WORKLOADS["lic_wh"]
    x = WL.gen_x(w, T=16)
    x[[0, 7, 15]] = 0.0
    c = IntCase(w, 16, 256, x=x)
    y = check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))
    g = c.gpu_constants()
    bias_only = O.int_forward(np.zeros((1, w.d_in), dtype=np.int16), g)["y_int"][0]
    for r in (0, 7, 15):
        assert np.array_equal(y[r], bias_only)


def test_wh_saturation():
    # a tenth of the calibrated output scale: most outputs clamp at +-127
    c = IntCase(WL.WORKLOADS["lic_wh"], 64, 256, s_y_factor=0.1)
    y = check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))
    assert (np.abs(y) == 127).mean() > 0.2


def test_wh_empty_batch():
    c = IntCase(WL.WORKLOADS["lic_wh"], 2, 256)
    Y = hq.int_linear(c.desc, c.prep, c.X[:0])
    assert Y.shape == (0, 256)


def test_wh_full_size():
    # lic_wh at its full 12288 tokens (the launch the benchmark times), every row
    w = WL.WORKLOADS["lic_wh"]
    c = IntCase(w, w.T, 256)
    check_constants(c)
    check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))


# ---- double-Hadamard layers

@pytest.mark.parametrize("m", [256, 1])
def test_dh_lic_first_rows(m):
    # DH-to-DH (m = 256: the output in the next layer's H_256 basis) and
    # DH-to-WH (m = 1)
    c = IntCase(WL.WORKLOADS["lic_wh"], 300, m, side=hq.HQ_INT_DH, in_block=256)
    check_constants(c)
    y = check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))
    sq = O.sqnr_db(c.y_ref / c.s_y, y.astype(np.float64))
    own = O.sqnr_db(c.y_ref / c.s_y, O.int_forward(c.xi, c.ora)["y_int"].astype(np.float64))
    print(f"lic DH m={m}: output SQNR {sq:.2f} dB (oracle {own:.2f} dB)")
    assert abs(sq - own) < 0.05 and sq > 15


@pytest.mark.parametrize("T,d_in,d_out,k,m,dtype", [
    (1, 128, 128, 128, 128, "f32"),
    (3, 384, 136, 128, 8, "f32"),
    (77, 256, 264, 1, 8, "f32"),     # no input-side rotation
    (130, 1152, 512, 64, 64, "bf16"),
    (257, 2048, 1024, 2048, 256, "f32"),
])
def test_dh_ragged(T, d_in, d_out, k, m, dtype):
    w = WL.custom(600 + T, T, d_in, d_out, dtype=dtype, x_dist="laplace", n_outliers=3,
                  outlier=20.0, w_std=0.05)
    c = IntCase(w, T, m, side=hq.HQ_INT_DH, in_block=k)
    check_constants(c)
    check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))


def test_dh_full_size():
    w = WL.WORKLOADS["lic_wh"]
    c = IntCase(w, w.T, 256, side=hq.HQ_INT_DH, in_block=256)
    check_constants(c)
    check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))


def test_dh_wh_two_layer_chain():
    # a DH layer (input in H_256) handing its int8 output to a WH layer
    # (m = 1: no transform), whose output is in the original basis; the GPU
    # chain equals the oracle's chain on the GPU's constants, code for code
    w1 = WL.custom(700, 200, 256, 512, dtype="f32", x_dist="laplace", n_outliers=3, outlier=20.0,
                   w_std=0.05)
    c1 = IntCase(w1, 200, 1, side=hq.HQ_INT_DH, in_block=256)
    y1 = hq.int_linear(c1.desc, c1.prep, c1.X)
    rng = np.random.default_rng(5)
    w2 = rng.normal(0, 0.03, (256, 512)).astype(np.float32)
    b2 = rng.normal(0, 0.01, 256).astype(np.float32)
    y2f = c1.y_ref @ w2.astype(np.float64).T + b2
    s2 = float(np.float32(np.abs(y2f).max() / 127.0))
    d2 = hq.IntDesc(512, 256, 256, hq.F32, hq.HQ_INT_WH, 1)
    p2 = hq.int_prepare(d2, torch.from_numpy(w2).cuda(), torch.from_numpy(b2).cuda(), c1.s_y, s2)
    y2 = to_np(hq.int_linear(d2, p2, y1)).astype(np.int64)
    g1 = c1.gpu_constants()
    v2 = hq.int_views(d2, p2)
    g2 = {"qw": to_np(v2["w_codes"]).astype(np.int64), "b_int": to_np(v2["b_int"]).astype(np.int64),
          "mult": to_np(v2["mult"]).astype(np.int64), "shift": int(to_np(v2["shift"])[0]),
          "block": 256}
    q1 = O.int_forward(c1.xi, g1)["y_int"]
    q2 = O.int_forward(q1, g2)["y_int"].astype(np.int64)
    assert np.array_equal(y2, q2)
    assert O.sqnr_db(y2f / s2, y2.astype(np.float64)) > 15


@pytest.mark.parametrize("side,k,T,d_out", [(hq.HQ_INT_WH, 1, 77, 512), (hq.HQ_INT_DH, 256, 300, 256)])
def test_fused_layer_equals_requant_stage(side, k, T, d_out):
    # d_out a multiple of 256: int_linear runs GEMM and requantisation in one
    # kernel. The standalone requantisation stage fed the exact int32 products
    # (formed here on the host) gives the same codes.
    w = WL.custom(800 + T, T, 256, d_out, dtype="f32", x_dist="laplace", n_outliers=3,
                  outlier=20.0, w_std=0.05)
    c = IntCase(w, T, 256, side=side, in_block=k)
    y = to_np(hq.int_linear(c.desc, c.prep, c.X)).astype(np.int64)
    g = c.gpu_constants()
    acc = c.xi.astype(np.int64) @ g["qw"][:d_out].T
    ys = to_np(hq.int_requant(c.desc, c.prep, torch.from_numpy(acc.astype(np.int32)).cuda()))
    assert np.array_equal(y, ys.astype(np.int64))


# ---- activations between layers (Table I; Eq. (20)-(22); supplement Eq. (45)-(49))

WH, DH = hq.HQ_INT_WH, hq.HQ_INT_DH
NONE, RELU, SILU, GELU = (hq.HQ_INT_ACT_NONE, hq.HQ_INT_ACT_RELU, hq.HQ_INT_ACT_SILU,
                          hq.HQ_INT_ACT_GELU)


@pytest.mark.parametrize("side,k,act,m,post", [
    (WH, 1, RELU, 256, 1),      # WH-to-WH with ReLU
    (WH, 1, NONE, 256, 64),     # WH-to-DH, both transforms, identity
    (WH, 1, RELU, 256, 256),    # WH-to-DH with ReLU (multiplier bound 255)
    (WH, 1, SILU, 16, 32),      # WH-to-DH with SiLU (table)
    (WH, 1, GELU, 256, 256),    # WH-to-DH with GELU (table)
    (DH, 256, RELU, 1, 128),    # DH-to-DH with ReLU
    (DH, 64, GELU, 1, 1),       # DH-to-WH with GELU
])
def test_transition_lic_first_rows(side, k, act, m, post):
    c = IntCase(WL.WORKLOADS["lic_wh"], 300, m, side=side, in_block=k, act=act, post=post)
    check_constants(c)
    y = check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))
    sq = O.sqnr_db(c.y_ref / c.s_y, y.astype(np.float64))
    print(f"output SQNR {sq:.2f} dB against phi(layer) in the next basis")
    assert sq > 12


@pytest.mark.parametrize("T,d_in,d_out,side,k,act,m,post,dtype", [
    (77, 256, 136, WH, 1, GELU, 8, 8, "f32"),        # two-kernel path (d_out % 256 != 0)
    (130, 384, 264, WH, 1, RELU, 8, 8, "bf16"),
    (3, 128, 128, DH, 128, SILU, 1, 128, "f32"),
    (257, 256, 1024, WH, 1, SILU, 256, 64, "f32"),   # several 256-channel chunks per row
])
def test_transition_ragged(T, d_in, d_out, side, k, act, m, post, dtype):
    w = WL.custom(900 + T, T, d_in, d_out, dtype=dtype, x_dist="laplace", n_outliers=3,
                  outlier=20.0, w_std=0.05)
    c = IntCase(w, T, m, side=side, in_block=k, act=act, post=post)
    check_constants(c)
    check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))


@pytest.mark.parametrize("act", [RELU, GELU])
def test_transition_full_size(act):
    # lic_wh as a WH-to-DH layer at its full 12288 tokens, every row
    w = WL.WORKLOADS["lic_wh"]
    c = IntCase(w, w.T, 256, act=act, post=256)
    check_constants(c)
    check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))


@pytest.mark.parametrize("act,m,post", [(RELU, 256, 256), (SILU, 16, 8), (GELU, 1, 256)])
def test_transition_requant_stage_bit_exact(act, m, post):
    # the requantisation alone on wide int32 products against the oracle's
    # integer steps on the GPU's constants (z saturates on both sides of the
    # table for the wide inputs)
    c = IntCase(WL.WORKLOADS["lic_wh"], 4, m, act=act, post=post)
    g = c.gpu_constants()
    rng = np.random.default_rng(23)
    acc = rng.integers(-2 ** 27, 2 ** 27, (257, c.w.d_out), dtype=np.int64)
    acc[:3] = 0
    acc[3] = 2 ** 27 - 1
    acc[4:40] //= 2 ** 14           # a band of small products: unsaturated z
    y = to_np(hq.int_requant(c.desc, c.prep, torch.from_numpy(acc.astype(np.int32)).cuda()))
    u = (acc + g["b_int"][None, :]) * g["mult"][None, :]
    v = O.unnormalised_transform(u, m)
    if act == RELU:
        ref = np.clip(O.round_half_even_shift(O.unnormalised_transform(np.maximum(v, 0), post),
                                              g["shift"]), -127, 127)
    else:
        z = np.clip(O.round_half_even_shift(v, g["shift"]), -127, 127)
        w2 = O.unnormalised_transform(g["lut"][z + 127] * g["mult_in"], post)
        ref = np.clip(O.round_half_even_shift(w2, g["shift_in"]), -127, 127)
    assert np.array_equal(y.astype(np.int64), ref)


@pytest.mark.parametrize("act,d_out", [(RELU, 512), (GELU, 256)])
def test_fused_transition_equals_requant_stage(act, d_out):
    w = WL.custom(950, 77, 256, d_out, dtype="f32", x_dist="laplace", n_outliers=3,
                  outlier=20.0, w_std=0.05)
    c = IntCase(w, 77, 256, act=act, post=128)
    y = to_np(hq.int_linear(c.desc, c.prep, c.X)).astype(np.int64)
    g = c.gpu_constants()
    acc = c.xi.astype(np.int64) @ g["qw"][:d_out].T
    ys = to_np(hq.int_requant(c.desc, c.prep, torch.from_numpy(acc.astype(np.int32)).cuda()))
    assert np.array_equal(y, ys.astype(np.int64))


def test_wh_gelu_dh_two_layer_chain():
    # an integer MLP: a WH layer with GELU hands its int8 output to a DH layer
    # in that layer's H_256 basis (Table I, WH-to-DH: H_out before GELU, H_in
    # after it); the DH layer ends in the original basis (DH-to-WH). The GPU
    # chain equals the oracle's chain on the GPU's constants, code for code.
    w1 = WL.custom(960, 200, 256, 512, dtype="f32", x_dist="laplace", n_outliers=3, outlier=20.0,
                   w_std=0.05)
    c1 = IntCase(w1, 200, 256, act=GELU, post=256)
    y1 = hq.int_linear(c1.desc, c1.prep, c1.X)
    rng = np.random.default_rng(6)
    w2 = rng.normal(0, 0.03, (256, 512)).astype(np.float32)
    b2 = rng.normal(0, 0.01, 256).astype(np.float32)
    h1 = O.gelu(np.asarray(c1.x, np.float64) @ np.asarray(c1.weight, np.float64).T + c1.bias)
    y2f = h1 @ w2.astype(np.float64).T + b2
    s2 = float(np.float32(np.abs(y2f).max() / 127.0))
    d2 = hq.IntDesc(512, 256, 1, hq.F32, DH, 256)
    p2 = hq.int_prepare(d2, torch.from_numpy(w2).cuda(), torch.from_numpy(b2).cuda(), c1.s_y, s2)
    y2 = to_np(hq.int_linear(d2, p2, y1)).astype(np.int64)
    v2 = hq.int_views(d2, p2)
    g2 = {"qw": to_np(v2["w_codes"]).astype(np.int64), "b_int": to_np(v2["b_int"]).astype(np.int64),
          "mult": to_np(v2["mult"]).astype(np.int64), "shift": int(to_np(v2["shift"])[0]),
          "block": 1}
    q1 = O.int_forward(c1.xi, c1.gpu_constants())["y_int"]
    q2 = O.int_forward(q1, g2)["y_int"].astype(np.int64)
    assert np.array_equal(y2, q2)
    sq = O.sqnr_db(y2f / s2, y2.astype(np.float64))
    print(f"two-layer integer MLP (WH + GELU -> DH): output SQNR {sq:.2f} dB")
    assert sq > 12


# ---- padded orders (supplement Sec. VII-B Eq. (35)-(41), Sylvester orders)

@pytest.mark.parametrize("act,post", [(NONE, 1), (RELU, 256), (GELU, 256), (SILU, 1)])
def test_padded_wh_output(act, post):
    # 200 outputs under H_256: 256 accumulator channels, the first 200 kept
    w = WL.custom(970, 130, 256, 200, dtype="bf16", x_dist="laplace", n_outliers=3,
                  outlier=20.0, w_std=0.05)
    c = IntCase(w, 130, 256, act=act, post=post)
    assert c.desc.acc_width == 256 and c.desc.out_width == max(post, 200)
    check_constants(c)
    y = check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))
    assert y.shape == (130, c.desc.out_width)
    assert O.sqnr_db(c.y_ref / c.s_y, y.astype(np.float64)) > 12


@pytest.mark.parametrize("d_in,k,d_out,act,post", [(200, 256, 64, NONE, 1), (200, 256, 120, RELU, 128),
                                                  (640, 1024, 256, GELU, 1)])
def test_padded_dh_input(d_in, k, d_out, act, post):
    # the DH input of d_in channels padded to H_k (the previous layer's padded
    # output); the second case also pads its own output for the next DH layer,
    # the third runs the fused kernel (d_out 256) on a padded input
    w = WL.custom(980 + d_in, 77, d_in, d_out, dtype="f32", x_dist="laplace", n_outliers=3,
                  outlier=20.0, w_std=0.05)
    c = IntCase(w, 77, 1, side=DH, in_block=k, act=act, post=post)
    assert c.desc.x_width == k
    check_constants(c)
    y = check_outputs(c, hq.int_linear(c.desc, c.prep, c.X))
    assert y.shape == (77, c.desc.out_width)


def test_padded_requant_stage_bit_exact():
    c = IntCase(WL.custom(990, 4, 256, 200, dtype="f32", x_dist="laplace"), 4, 256, act=RELU,
                post=256)
    g = c.gpu_constants()
    rng = np.random.default_rng(29)
    acc = rng.integers(-2 ** 27, 2 ** 27, (129, 256), dtype=np.int64)
    acc[:2] = 0
    y = to_np(hq.int_requant(c.desc, c.prep, torch.from_numpy(acc.astype(np.int32)).cuda()))
    u = (acc + g["b_int"][None, :]) * g["mult"][None, :]
    v = np.maximum(O.unnormalised_transform(u, 256)[:, :200], 0)
    v = np.concatenate([v, np.zeros((129, 56), np.int64)], axis=1)
    ref = np.clip(O.round_half_even_shift(O.unnormalised_transform(v, 256), g["shift"]), -127, 127)
    assert y.shape == (129, 256) and np.array_equal(y.astype(np.int64), ref)


def test_padded_wh_relu_dh_chain():
    # Table I, WH-to-DH across padded orders: a WH layer (200 outputs under
    # H_256) with ReLU hands 256 codes in the next layer's padded H_256 basis
    # to a DH layer whose 200 input channels are padded to 256; the GPU chain
    # equals the oracle's chain on the GPU's constants, code for code
    w1 = WL.custom(995, 120, 256, 200, dtype="f32", x_dist="laplace", n_outliers=3, outlier=20.0,
                   w_std=0.05)
    c1 = IntCase(w1, 120, 256, act=RELU, post=256)
    y1 = hq.int_linear(c1.desc, c1.prep, c1.X)
    assert tuple(y1.shape) == (120, 256)
    rng = np.random.default_rng(7)
    w2 = rng.normal(0, 0.05, (136, 200)).astype(np.float32)
    b2 = rng.normal(0, 0.01, 136).astype(np.float32)
    h1 = np.maximum(np.asarray(c1.x, np.float64) @ np.asarray(c1.weight, np.float64).T + c1.bias, 0)
    y2f = h1 @ w2.astype(np.float64).T + b2
    s2 = float(np.float32(np.abs(y2f).max() / 127.0))
    d2 = hq.IntDesc(200, 136, 1, hq.F32, DH, 256)
    p2 = hq.int_prepare(d2, torch.from_numpy(w2).cuda(), torch.from_numpy(b2).cuda(), c1.s_y, s2)
    y2 = to_np(hq.int_linear(d2, p2, y1)).astype(np.int64)
    v2 = hq.int_views(d2, p2)
    g2 = {"qw": to_np(v2["w_codes"]).astype(np.int64), "b_int": to_np(v2["b_int"]).astype(np.int64),
          "mult": to_np(v2["mult"]).astype(np.int64), "shift": int(to_np(v2["shift"])[0]),
          "block": 1, "d_out": 136}
    q1 = O.int_forward(c1.xi, c1.gpu_constants())["y_int"]
    assert np.array_equal(to_np(y1).astype(np.int64), q1.astype(np.int64))
    q2 = O.int_forward(q1, g2)["y_int"].astype(np.int64)
    assert np.array_equal(y2, q2)
    sq = O.sqnr_db(y2f / s2, y2.astype(np.float64))
    print(f"padded integer MLP (WH 200 under H_256 + ReLU -> DH 200 padded to 256): SQNR {sq:.2f} dB")
    assert sq > 12
