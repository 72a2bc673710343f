"""GPU parity of per-channel centring (descriptor center = 2): the "one added
token" reading of HadaNorm Eq. (1), mu = mean over the call's tokens of each
channel of X diag(1/sigma) H and b~ = b + mu W~, against the CPU oracle.

Cases: every workload's shape with its centring switched to the per-channel
mode, on its first 300 tokens (square4k is the workload whose channels carry
different means), plus equal tokens (X~ = 0) and square4k at full size on
sampled tokens. Tolerances are those of tests/parity.py; the statistics
(the channel mean and the corrected bias) are checked at float32
accumulation accuracy.
"""
import dataclasses

import numpy as np
import pytest
import torch

import hadamard_rotated_bit_amd as hq
from hadamard_rotated_bit_amd import workloads as WL
from oracle import hq_oracle as O
from parity import (XT_TOL, Y_TOL, Case, check_codes, codes_np, desc_for, rel_fro, tdev, to_np)

pytestmark = pytest.mark.gpu

_CASES = {}


def chan_case(name: str, T: int = 300) -> Case:
    key = (name, T)
    if key not in _CASES:
        print(f"\n[case] channel-centred {name} T={T}", flush=True)
        w = dataclasses.replace(WL.WORKLOADS[name], center=O.CENTER_CHANNEL)
        _CASES[key] = Case(w, T)
    return _CASES[key]


@pytest.mark.parametrize("name", WL.ORDER)
def test_channel_statistics(name):
    c = chan_case(name)
    mean, bias_eff = hq.channel_center(c.desc, c.prep, c.X)
    mean, bias_eff = to_np(mean).astype(np.float64), to_np(bias_eff).astype(np.float64)
    xs = c.x.astype(np.float64)
    assert np.all(np.abs(mean - xs.mean(axis=0)) <= 1e-5 * (np.abs(xs).mean(axis=0) + 1e-30))
    ref_bias = c.ora["bias_eff"]
    bound = 1e-4 * (np.abs(c.bias) + np.abs(c.weight.astype(np.float64)) @ np.abs(xs).mean(axis=0))
    d = c.w.d_out
    assert np.all(np.abs(bias_eff[:d] - ref_bias) <= bound)
    assert not bias_eff[d:].any()
    # the oracle's b + mu W~ is the mean token through the original weight
    np.testing.assert_allclose(ref_bias - c.bias, c.weight.astype(np.float64) @ xs.mean(axis=0),
                               rtol=1e-9, atol=1e-9 * np.abs(ref_bias).max())


@pytest.mark.parametrize("name", WL.ORDER)
def test_channel_transform(name):
    c = chan_case(name)
    xt, _ = hq.act_transform(c.desc, c.prep, c.X)
    xt = to_np(xt).astype(np.float64)
    o = c.ora
    rows = np.linalg.norm(xt - o["xt"], axis=1) / np.maximum(np.linalg.norm(o["xt"], axis=1), 1e-300)
    assert rows.max() <= XT_TOL, rows.max()
    # every channel of X~ sums to zero over the tokens (to float32 accuracy)
    assert np.all(np.abs(xt.sum(axis=0)) <= 1e-4 * np.abs(o["y"]).sum(axis=0) + 1e-30)


@pytest.mark.parametrize("name", WL.ORDER)
def test_channel_codes_and_output(name):
    c = chan_case(name)
    o = c.ora
    codes, s_x, mean, U = hq.act_quantize(c.desc, c.prep, c.X)
    ratio = np.divide(o["xt"], o["s_x"][:, None], out=np.zeros_like(o["xt"]),
                      where=o["s_x"][:, None] > 0)
    flips = check_codes(codes_np(c.desc, codes, c.T), o["qa"], ratio, "activation codes")
    print(f"{name}: {flips} flipped codes of {o['qa'].size}")
    np.testing.assert_allclose(to_np(s_x), o["s_x"], rtol=1e-5)
    Y = hq.quant_linear(c.desc, c.prep, c.X)
    err = rel_fro(to_np(Y), o["y_out"])
    print(f"{name}: rel Frobenius error {err:.3e}")
    assert err <= Y_TOL, err
    # the staged path (statistics, activation stage, GEMM + epilogue) gives the same bits
    _, bias_eff = hq.channel_center(c.desc, c.prep, c.X)
    Y2 = hq.gemm_dequant(c.desc, c.prep, codes, s_x, bias_eff, U)
    assert torch.equal(Y, Y2)


@pytest.mark.parametrize("name,T", [("dit_fc1", 4), ("square4k", 1), ("tiny", 2), ("lic_dh", 2)])
def test_channel_equal_tokens(name, T):
    # identical tokens centre to X~ = 0: codes and scales are 0 and Y is the
    # unquantised layer b + x W (up to the float32 bias product and the output
    # dtype). The token counts keep the float32 mean of the equal values exact
    # (bf16 inputs: 4 rows; float32 inputs: 1 or 2 rows).
    w = dataclasses.replace(WL.WORKLOADS[name], center=O.CENTER_CHANNEL)
    x = np.tile(WL.gen_x(w, T=1), (T, 1))
    c = Case(w, T, x=x)
    codes, s_x, _, _ = hq.act_quantize(c.desc, c.prep, c.X)
    assert not codes_np(c.desc, codes, T).any()
    assert not to_np(s_x).any()
    Y = to_np(hq.quant_linear(c.desc, c.prep, c.X))
    ref = O.round_to_dtype(O.exact_output(x, c.weight, c.bias), w.out_dtype)
    tol = 1e-5 if w.out_dtype == "f32" else Y_TOL   # bf16: a last-bit flip is allowed
    assert rel_fro(Y, ref) <= tol
    assert rel_fro(Y, c.ora["y_out"]) <= tol


def test_channel_full_size_sampled():
    # square4k at its full 8192 tokens: the channel mean over all of them, then
    # 64 sampled tokens through the oracle's steps with that mean
    w = dataclasses.replace(WL.WORKLOADS["square4k"], center=O.CENTER_CHANNEL)
    print(f"\n[case] channel-centred full-size square4k T={w.T}", flush=True)
    desc = desc_for(w)
    x = WL.gen_x(w)
    weight, bias = WL.gen_weight(w), WL.gen_bias(w)
    X = tdev(x, w.dtype)
    prep = hq.prepare(desc, tdev(weight, w.dtype), torch.from_numpy(bias).cuda())
    Y = hq.quant_linear(desc, prep, X)
    codes, s_x, _, _ = hq.act_quantize(desc, prep, X)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(np.arange(8, w.T - 8), 48, replace=False),
                                     np.arange(w.T - 8, w.T)]))
    idx = torch.from_numpy(rows).cuda()
    y_s, c_s, sx_s = to_np(Y[idx]), codes_np(desc, codes, w.T, rows), to_np(s_x[idx])
    del Y, codes, X

    ones = np.ones(w.d_in)
    prepd = O.prepare_weights(weight, ones, w.block, w.w_bits)
    mu_c = O.rotate(x.astype(np.float64).mean(axis=0)[None, :], w.block)[0]
    xt = O.rotate(x[rows].astype(np.float64), w.block) - mu_c[None, :]
    qa, sx = O.quantize_rows(xt, w.a_bits)
    yf = O.dequant_output(O.int_gemm(qa, prepd["qw"]), sx, prepd["s_w"],
                          O.channel_bias(bias, prepd["wt"], mu_c), np.zeros(len(rows)), prepd["c"])
    err = rel_fro(y_s, O.round_to_dtype(yf, w.out_dtype))
    print(f"square4k channel-centred: sampled rel Frobenius error {err:.3e}")
    assert err <= Y_TOL, err
    ratio = np.divide(xt, sx[:, None], out=np.zeros_like(xt), where=sx[:, None] > 0)
    check_codes(c_s, qa, ratio, "activation codes (sampled)")
    np.testing.assert_allclose(sx_s, sx, rtol=1e-5)
