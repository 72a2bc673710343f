"""Pins of the C++17 CPU oracle (oracle/hq_oracle.cpp) against the pinned
float64 NumPy oracle (oracle/hq_oracle.py), on the CPU.

The two share no code: the C++ oracle evaluates the rotation as the signed
sums of HaTQ Eq. (8) with the popcount entries of the Sylvester matrix, the
NumPy oracle as a dense product with the doubling construction. Codes,
accumulators, scales and means must agree exactly; float values to the
float64 rounding of the two summation orders.
"""
import numpy as np
import pytest

from hadamard_rotated_bit_amd import workloads as WL
from oracle import cpp as C
from oracle import hq_oracle as O


@pytest.fixture(scope="module", autouse=True)
def built():
    C.build()
    yield


@pytest.mark.parametrize("block", [1, 2, 8, 64, 256])
def test_rotation_matches_dense_definition(block):
    rng = np.random.default_rng(block)
    x = rng.standard_normal((5, 512))
    np.testing.assert_allclose(C.rotate(x, block), O.rotate(x, block), rtol=0, atol=1e-12)
    # rows of H_B: orthonormal and symmetric
    h = C.rotate(np.eye(block), block)
    np.testing.assert_allclose(h @ h.T, np.eye(block), atol=1e-13)
    np.testing.assert_allclose(h, h.T, atol=0)


def test_rotation_rejects_bad_block():
    with pytest.raises(ValueError):
        C.rotate(np.zeros((2, 96)), 64)


def check_codes_equal(got, want, v):
    """Equal codes, except (never seen in practice) where the float64 quotient
    sits within 1e-9 of a half-integer in the NumPy oracle's arithmetic."""
    d = np.asarray(got, dtype=np.int64) - np.asarray(want, dtype=np.int64)
    bad = d != 0
    if bad.any():
        av = np.abs(np.asarray(v)[bad])
        assert np.abs(d).max() == 1
        assert np.abs(av - np.floor(av) - 0.5).max() < 1e-9


CASES = [("tiny", 64), ("dit_fc1", 48), ("square4k", 12), ("square4k_nc", 12), ("lic_dh", 64),
         ("flux_proj", 24)]


@pytest.mark.parametrize("name,rows", CASES)
def test_layer_matches_numpy_oracle(name, rows):
    w = WL.WORKLOADS[name]
    x = WL.gen_x(w, T=rows)
    weight, bias = WL.gen_weight(w), WL.gen_bias(w)
    l1, l2 = WL.gen_lowrank(w)
    # a sample of output channels (each channel's codes, scale and c depend
    # on its own weight row only): the first 32 and 32 seeded others
    if w.d_out > 64:
        sel = np.concatenate([np.arange(32), np.sort(np.random.default_rng(9).choice(
            np.arange(32, w.d_out), 32, replace=False))])
        weight, bias = weight[sel], bias[sel]
        l2 = None if l2 is None else l2[:, sel]
    sigma = (O.smoothing_scales(WL.gen_x(w, T=min(w.T, 256)), WL.gen_weight(w), w.alpha)
             if w.alpha is not None else np.ones(w.d_in))
    pn = O.prepare_weights(weight, sigma, w.block, w.w_bits)
    pc = C.prepare_weights(weight, sigma, w.block, w.w_bits)
    check_codes_equal(pc["qw"], pn["qw"], pn["wt"] / np.where(pn["s_w"] > 0, pn["s_w"], 1)[:, None])
    np.testing.assert_allclose(pc["s_w"], pn["s_w"], rtol=1e-13)
    np.testing.assert_allclose(pc["c"], pn["c"], rtol=0, atol=1e-12 * np.abs(pn["wt"]).sum(axis=1).max())
    rn = O.quant_linear(x, pn, bias, sigma, block=w.block, a_bits=w.a_bits, center=int(w.center),
                        l1=l1, l2=l2, out_dtype=w.out_dtype)
    # the C++ side runs on its own prepared weights (equal codes, asserted above)
    rc = C.quant_linear(x, pc, bias, sigma, block=w.block, a_bits=w.a_bits,
                        center=int(w.center), l1=l1, l2=l2, out_dtype=w.out_dtype)
    ratio = np.divide(rn["xt"], rn["s_x"][:, None], out=np.zeros_like(rn["xt"]),
                      where=rn["s_x"][:, None] > 0)
    check_codes_equal(rc["qa"], rn["qa"], ratio)
    np.testing.assert_allclose(rc["s_x"], rn["s_x"], rtol=1e-13)
    np.testing.assert_allclose(rc["mu"], rn["mu"], rtol=0,
                               atol=1e-13 * np.abs(rn["y"]).max())
    if np.array_equal(rc["qa"], rn["qa"]) and np.array_equal(pc["qw"], pn["qw"]):
        np.testing.assert_array_equal(rc["acc"], rn["acc"])     # exact integer products
    # outputs: equal up to the last bit of the output type, where the two
    # float64 summation orders straddle a rounding boundary
    yn, yc = rn["y_out"], rc["y_out"]
    ulp = np.abs(yn) * (2.0 ** -7 if w.out_dtype == "bf16" else 2.0 ** -23) + 1e-300
    diff = np.abs(yc - yn)
    assert np.all(diff <= ulp), diff.max()
    assert (diff > 0).mean() <= 1e-3


def test_identity_codes_return_the_other_operand():
    # special case of the integer product: with one activation code 1 at
    # channel k and scales of 1, acc[:, j] is the weight code qw[j, k]
    rng = np.random.default_rng(3)
    d_in, d_out = 16, 8
    weight = rng.standard_normal((d_out, d_in))
    pc = C.prepare_weights(weight, None, 1, 4)
    x = np.zeros((d_in, d_in))
    np.fill_diagonal(x, 1.0)
    r = C.quant_linear(x, pc, None, None, block=1, a_bits=4, center=0)
    np.testing.assert_array_equal(r["qa"], 7 * np.eye(d_in, dtype=np.int16))
    np.testing.assert_array_equal(r["acc"], 7 * pc["qw"].T.astype(np.int64))


def test_bad_arguments_are_rejected():
    pc = C.prepare_weights(np.ones((8, 16)), None, 16, 4)
    with pytest.raises(ValueError):
        C.quant_linear(np.ones((2, 16)), pc, None, None, block=16, a_bits=5, center=1)
    with pytest.raises(ValueError):
        C.quant_linear(np.ones((2, 16)), pc, None, None, block=16, a_bits=4, center=2)
    with pytest.raises(ValueError):
        C.prepare_weights(np.ones((8, 16)), None, 3, 4)
