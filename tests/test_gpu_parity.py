"""GPU parity: every stage of the HIP path against the CPU oracle, through the C ABI.

Each workload runs on its first 300 tokens (several K1 waves, two GEMM row
tiles plus a ragged tail) at its full d_in and d_out; tolerances are those
of tests/parity.py.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_bit_amd as hq
from hadamard_rotated_bit_amd import workloads as WL
from oracle import hq_oracle as O
from parity import (ENGINE_CASES, MAX_FLIP_FRAC, XT_TOL, Y_TOL, case_id, check_codes, codes_dev,
                    codes_np, rel_fro, small_case, tdev, to_np)

pytestmark = pytest.mark.gpu
NAMES = WL.PARITY_ORDER


@pytest.mark.parametrize("name", [n for n in NAMES if WL.WORKLOADS[n].alpha is not None])
def test_sigma(name):
    c = small_case(name)
    amax = hq.channel_absmax(c.desc, c.X)
    np.testing.assert_array_equal(to_np(amax), np.abs(c.x).max(axis=0).astype(np.float32))
    sig = hq.sigma(c.desc, amax, c.W, c.w.alpha)
    err = np.abs(to_np(sig).astype(np.float64) / c.sigma64 - 1).max()
    assert err <= 1e-6, err


@pytest.mark.parametrize("ec", ENGINE_CASES, ids=case_id)
def test_weight_prepare(ec):
    name = ec[0]
    c = small_case(name, gemm=ec[1])
    v = hq.prepared_views(c.desc, c.prep)
    o = c.ora
    qmax = 2 ** (c.w.w_bits - 1) - 1
    ratio = np.divide(o["wt"], o["s_w"][:, None], out=np.zeros_like(o["wt"]),
                      where=o["s_w"][:, None] > 0)
    wc = codes_np(c.desc, v["w_codes"], c.desc.d_out)
    check_codes(wc, o["qw"], ratio, "weight codes")
    assert np.abs(wc).max() <= qmax
    np.testing.assert_allclose(to_np(v["s_w"]), o["s_w"], rtol=1e-5)
    cerr = np.abs(to_np(v["c"]) - o["c"]) / np.abs(o["wt"]).sum(axis=1)
    assert cerr.max() <= 1e-5, cerr.max()
    np.testing.assert_array_equal(to_np(v["bias"]), c.bias)
    if c.desc.smooth:
        np.testing.assert_allclose(to_np(v["sigma_inv"]), 1.0 / c.sigma32.astype(np.float64),
                                   rtol=1e-6)


@pytest.mark.parametrize("name", NAMES)
def test_activation_transform(name):
    c = small_case(name)
    xt, mu = hq.act_transform(c.desc, c.prep, c.X)
    xt, mu = to_np(xt), to_np(mu)
    o = c.ora
    rows = np.linalg.norm(xt - o["xt"], axis=1) / np.maximum(np.linalg.norm(o["xt"], axis=1), 1e-300)
    assert rows.max() <= XT_TOL, rows.max()
    rms = np.sqrt(np.mean(o["y"] ** 2, axis=1))
    assert np.all(np.abs(mu - o["mu"]) <= XT_TOL * rms)
    if c.desc.center:   # centred rows sum to zero (to float32 accuracy)
        assert np.all(np.abs(xt.astype(np.float64).sum(axis=1))
                      <= 1e-5 * np.abs(o["xt"]).sum(axis=1))


@pytest.mark.parametrize("ec", ENGINE_CASES, ids=case_id)
def test_activation_codes(ec):
    name = ec[0]
    c = small_case(name, gemm=ec[1])
    codes, s_x, mu, U = hq.act_quantize(c.desc, c.prep, c.X)
    o = c.ora
    ratio = np.divide(o["xt"], o["s_x"][:, None], out=np.zeros_like(o["xt"]),
                      where=o["s_x"][:, None] > 0)
    flips = check_codes(codes_np(c.desc, codes, c.T), o["qa"], ratio, "activation codes")
    print(f"{name}: {flips} activation code flips of {o['qa'].size}")
    np.testing.assert_allclose(to_np(s_x), o["s_x"], rtol=1e-5)
    rms = np.sqrt(np.mean(o["y"] ** 2, axis=1))
    assert np.all(np.abs(to_np(mu) - o["mu"]) <= XT_TOL * rms)
    if c.desc.rank:
        u = to_np(U)
        err = np.linalg.norm(u - o["u"], axis=1) / np.linalg.norm(o["u"], axis=1)
        assert err.max() <= 1e-4, err.max()


@pytest.mark.parametrize("ec", ENGINE_CASES, ids=case_id)
def test_gemm_bit_exact(ec):
    name = ec[0]
    c = small_case(name, gemm=ec[1])
    o = c.ora
    a = codes_dev(c.desc, o["qa"])
    w = codes_dev(c.desc, o["qw"])
    acc = hq.gemm_i32(c.desc, a, w, c.T, c.desc.d_out)
    np.testing.assert_array_equal(to_np(acc).astype(np.int64), o["acc"])


@pytest.mark.parametrize("ec", ENGINE_CASES, ids=case_id)
def test_output(ec):
    name = ec[0]
    c = small_case(name, gemm=ec[1])
    Y = hq.quant_linear(c.desc, c.prep, c.X)
    err = rel_fro(to_np(Y), c.ora["y_out"])
    print(f"{name}: rel Frobenius error {err:.3e}")
    assert err <= Y_TOL, err
    # the stage entry points reproduce the fused call bit for bit
    codes, s_x, mu, U = hq.act_quantize(c.desc, c.prep, c.X)
    Y2 = hq.gemm_dequant(c.desc, c.prep, codes, s_x, mu, U)
    assert torch.equal(Y, Y2)
    # deterministic: a second call is bitwise identical
    assert torch.equal(Y, hq.quant_linear(c.desc, c.prep, c.X))


@pytest.mark.parametrize("ec", ENGINE_CASES, ids=case_id)
def test_output_with_oracle_codes_is_tight(ec):
    # Epilogue check: feeding the oracle's own codes/scales/mu (and U) through the GEMM
    # + dequant epilogue reproduces the oracle's output up to float32 epilogue rounding.
    c = small_case(ec[0], gemm=ec[1])
    o = c.ora
    codes = codes_dev(c.desc, o["qa"])
    s_x = torch.from_numpy(o["s_x"].astype(np.float32)).cuda()
    mu = torch.from_numpy(o["mu"].astype(np.float32)).cuda()
    U = None if o["u"] is None else torch.from_numpy(o["u"].astype(np.float32)).cuda()
    # substitute the oracle's weight codes too (in a copy of the blob), so
    # only the epilogue differs even where a weight code sits at a tie
    prep = c.prep.clone()
    L = hq.layout(c.desc)
    wc = codes_dev(c.desc, o["qw"])
    prep[L.w_codes:L.w_codes + wc.numel()].copy_(wc)
    assert np.array_equal(codes_np(c.desc, hq.prepared_views(c.desc, prep)["w_codes"],
                                   c.desc.d_out), o["qw"])
    Y = hq.gemm_dequant(c.desc, prep, codes, s_x, mu, U)
    y_ref = o["y_full"]
    tol = 2e-6 if c.w.out_dtype == "f32" else 8e-3
    err = np.abs(to_np(Y) - y_ref).max() / np.abs(y_ref).max()
    assert err <= tol, err
