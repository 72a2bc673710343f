"""GPU parity of the weight-only Hadamard (WH) layer with integer
requantisation (HaTQ Sec. IV-B Eq. (15)-(22), supplement Eq. (40)-(44))
against the CPU oracle.

The online path is integer arithmetic, so it is held to bit-exactness: the
GPU's output codes must equal the oracle's integer path run on the same
constants (read back from the GPU's prepared blob). The offline constants are
decided in float32 (W-bar, s_w) and float64 (the rest) on the GPU and in
float64 by the oracle, so they are compared to the oracle's own constants
with rounding-aware tolerances: W-bar per row to 2e-6, codes equal except
near-ties (tests/parity.py), multipliers and bias codes equal except where the
oracle's value lies within the float32 uncertainty of a half-integer, the
shift equal. Cases: the lic_wh workload (12288 x 256 -> 256, H_256) on its
first 300 tokens and at full size; ragged token counts and widths; blocks 1 to
256; bf16 weights; zero rows; saturated outputs.
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


def calibrate(x, weight, bias):
    """Static per-tensor scales (the inputs of the offline step): s_x from the
    input, s_y from the float layer's output, both rounded to float32."""
    s_x = np.float32(np.abs(x).max() / 127.0)
    y = np.asarray(x, dtype=np.float64) @ np.asarray(weight, dtype=np.float64).T + bias
    s_y = np.float32(np.abs(y).max() / 127.0)
    return float(s_x), float(s_y)


class WhCase:
    def __init__(self, w: WL.Workload, T: int, m: int, x=None, s_y_factor: float = 1.0):
        print(f"\n[case] WH {w.name} T={T} {w.d_in}->{w.d_out} m={m} {w.dtype}", flush=True)
        self.w, self.T, self.m = w, T, m
        self.x = WL.gen_x(w, T=T) if x is None else x
        self.weight = WL.gen_weight(w)
        self.bias = WL.gen_bias(w)
        self.s_x, s_y = calibrate(self.x if T else np.ones((1, w.d_in)), self.weight, self.bias)
        self.s_y = float(np.float32(s_y * s_y_factor))
        self.desc = hq.WhDesc(w.d_in, w.d_out, m, DT[w.dtype])
        self.xi = O.quantize_static(self.x, self.s_x)
        self.ora = O.wh_prepare(self.weight, self.bias, self.s_x, self.s_y, m)
        self.prep = hq.wh_prepare(self.desc, tdev(self.weight, w.dtype),
                                  torch.from_numpy(self.bias).cuda(), self.s_x, self.s_y)
        self.X = torch.from_numpy(self.xi.astype(np.int8)).cuda()

    def gpu_constants(self):
        v = hq.wh_views(self.desc, self.prep)
        return {"qw": to_np(v["w_codes"]).astype(np.int64), "b_int": to_np(v["b_int"]).astype(np.int64),
                "mult": to_np(v["mult"]).astype(np.int64), "shift": int(to_np(v["shift"])[0]),
                "block": self.m, "s_w": to_np(v["s_w"]).astype(np.float64),
                "wbar": to_np(v["wbar"]).astype(np.float64)}


def check_constants(c: WhCase):
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
    t = o["rho"] * 2.0 ** o["shift"]
    d = g["mult"] - o["mult"]
    assert np.abs(d).max() <= 1
    if d.any():
        win = 4e-6 * np.abs(t[d != 0]) + 1e-9
        assert np.all(np.abs(np.abs(t[d != 0] - np.floor(t[d != 0])) - 0.5) <= win)
    # bias codes: round(b-bar / s_A)
    s_a = c.s_x * o["s_w"]
    tb = np.divide(o["bbar"], s_a, out=np.zeros_like(s_a), where=s_a > 0)
    db = g["b_int"] - o["b_int"]
    assert np.abs(db).max() <= 1
    if db.any():
        win = 4e-6 * np.abs(tb[db != 0]) + 1e-9
        assert np.all(np.abs(np.abs(tb[db != 0] - np.floor(tb[db != 0])) - 0.5) <= win)
    return g


def check_outputs(c: WhCase, Y):
    g = c.gpu_constants()
    y = to_np(Y).astype(np.int64)
    # bit-exact against the oracle's integer path on the GPU's constants
    ref = O.wh_forward_int(c.xi, g)["y_int"].astype(np.int64)
    assert np.array_equal(y, ref), np.argwhere(y != ref)[:5]
    # and within one code of the oracle's own constants, nearly everywhere equal
    own = O.wh_forward_int(c.xi, c.ora)["y_int"].astype(np.int64)
    diff = np.abs(y - own)
    if diff.size:
        assert diff.max() <= 1
        assert (diff > 0).mean() <= 1e-3, (diff > 0).mean()
    return y


def test_wh_lic_first_rows():
    c = WhCase(WL.WORKLOADS["lic_wh"], 300, 256)
    check_constants(c)
    Y = hq.wh_linear(c.desc, c.prep, c.X)
    y = check_outputs(c, Y)
    exact = (c.x.astype(np.float64) @ c.weight.astype(np.float64).T + c.bias) / c.s_y
    sq = O.sqnr_db(exact, y.astype(np.float64))
    own = O.sqnr_db(exact, O.wh_forward_int(c.xi, c.ora)["y_int"].astype(np.float64))
    print(f"lic_wh: output SQNR {sq:.2f} dB against the float layer (oracle {own:.2f} dB)")
    # the activation keeps its original basis and one per-tensor scale, so the
    # x30 outlier channels coarsen its grid; int8 still reaches ~20 dB here
    assert abs(sq - own) < 0.05 and sq > 15


def test_wh_requant_stage_bit_exact():
    # the requantisation alone on wide int32 products (beyond what 8-bit codes
    # produce), against the oracle's integer steps on the GPU's constants
    c = WhCase(WL.WORKLOADS["lic_wh"], 4, 256)
    g = c.gpu_constants()
    rng = np.random.default_rng(21)
    acc = rng.integers(-2 ** 27, 2 ** 27, (257, c.w.d_out), dtype=np.int64)
    acc[:3] = 0
    acc[3] = 2 ** 27 - 1
    y = to_np(hq.wh_requant(c.desc, c.prep, torch.from_numpy(acc.astype(np.int32)).cuda()))
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
    c = WhCase(w, T, m)
    check_constants(c)
    check_outputs(c, hq.wh_linear(c.desc, c.prep, c.X))


def test_wh_zero_rows_pass_the_bias():
    w = WL.WORKLOADS["lic_wh"]
    x = WL.gen_x(w, T=16)
    x[[0, 7, 15]] = 0.0
    c = WhCase(w, 16, 256, x=x)
    y = check_outputs(c, hq.wh_linear(c.desc, c.prep, c.X))
    g = c.gpu_constants()
    bias_only = O.wh_forward_int(np.zeros((1, w.d_in), dtype=np.int16), g)["y_int"][0]
    for r in (0, 7, 15):
        assert np.array_equal(y[r], bias_only)


def test_wh_saturation():
    # a tenth of the calibrated output scale: most outputs clamp at +-127
    c = WhCase(WL.WORKLOADS["lic_wh"], 64, 256, s_y_factor=0.1)
    y = check_outputs(c, hq.wh_linear(c.desc, c.prep, c.X))
    assert (np.abs(y) == 127).mean() > 0.2


def test_wh_empty_batch():
    c = WhCase(WL.WORKLOADS["lic_wh"], 2, 256)
    Y = hq.wh_linear(c.desc, c.prep, c.X[:0])
    assert Y.shape == (0, 256)


def test_wh_full_size():
    # lic_wh at its full 12288 tokens (the launch the benchmark times), every row
    w = WL.WORKLOADS["lic_wh"]
    c = WhCase(w, w.T, 256)
    check_constants(c)
    check_outputs(c, hq.wh_linear(c.desc, c.prep, c.X))
