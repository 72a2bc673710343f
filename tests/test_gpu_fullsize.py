"""GPU parity at the workloads' full sizes, in the launch configurations the
benchmark times, checked on sampled tokens the oracle computes one by one.

* Y and the activation codes / scales / means of 64 sampled tokens (first 8,
  last 8 and 48 seeded random ones) against the oracle on those tokens.
* The integer GEMM at full size on seeded random codes: every sampled row of
  the int32 accumulators is bit-exact against the oracle's integer product.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_bit_amd as hq
from hadamard_rotated_bit_amd import workloads as WL
from oracle import hq_oracle as O
from parity import (ENGINE_CASES, Y_TOL, case_id, check_codes, codes_dev, codes_np, desc_for, rel_fro,
                    tdev, to_np)

pytestmark = pytest.mark.gpu


def sample_rows(T, n=64, seed=7):
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(8, T - 8), size=n - 16, replace=False)
    return np.unique(np.concatenate([np.arange(8), mid, np.arange(T - 8, T)]))


@pytest.mark.parametrize("name", WL.PARITY_ORDER)
def test_full_size_sampled(name):
    w = WL.WORKLOADS[name]
    print(f"\n[case] full-size {name} T={w.T}", flush=True)
    desc = desc_for(w)
    x = WL.gen_x(w)
    weight, bias = WL.gen_weight(w), WL.gen_bias(w)
    l1, l2 = WL.gen_lowrank(w)
    sig = None
    if w.alpha is not None:
        sig = O.smoothing_scales(x, weight, w.alpha).astype(np.float32).astype(np.float64)
    X = tdev(x, w.dtype)
    prep = hq.prepare(desc, tdev(weight, w.dtype), torch.from_numpy(bias).cuda(),
                      None if sig is None else torch.from_numpy(sig.astype(np.float32)).cuda(),
                      None if l1 is None else tdev(l1, w.dtype),
                      None if l2 is None else tdev(l2, w.dtype))
    Y = hq.quant_linear(desc, prep, X)
    codes, s_x, mu, U = hq.act_quantize(desc, prep, X)
    torch.cuda.synchronize()
    rows = sample_rows(w.T)
    idx = torch.from_numpy(rows).cuda()
    y_s, c_s = to_np(Y[idx]), codes_np(desc, codes, w.T, rows)
    sx_s, mu_s = to_np(s_x[idx]), to_np(mu[idx])
    del Y, codes, X

    ora = O.run(x[rows], weight, bias, block=w.block, a_bits=w.a_bits, w_bits=w.w_bits,
                center=int(w.center), sigma=sig, l1=l1, l2=l2, out_dtype=w.out_dtype)
    err = rel_fro(y_s, ora["y_out"])
    print(f"{name}: sampled rel Frobenius error {err:.3e}")
    assert err <= Y_TOL, err
    ratio = np.divide(ora["xt"], ora["s_x"][:, None], out=np.zeros_like(ora["xt"]),
                      where=ora["s_x"][:, None] > 0)
    check_codes(c_s, ora["qa"], ratio, "activation codes (sampled)")
    np.testing.assert_allclose(sx_s, ora["s_x"], rtol=1e-5)
    rms = np.sqrt(np.mean(ora["y"] ** 2, axis=1))
    assert np.all(np.abs(mu_s - ora["mu"]) <= 1e-5 * rms)


@pytest.mark.parametrize("ec", ENGINE_CASES, ids=case_id)
def test_full_size_gemm_bit_exact(ec):
    name = ec[0]
    w = WL.WORKLOADS[name]
    print(f"\n[case] full-size GEMM {name} {w.T}x{w.d_out}x{w.d_in} gemm={ec[1]}", flush=True)
    desc = desc_for(w, ec[1])
    qmax = 2 ** (w.a_bits - 1) - 1
    rng = np.random.default_rng(1234 + w.key)
    a = rng.integers(-qmax, qmax + 1, (w.T, w.d_in), dtype=np.int8)
    b = rng.integers(-qmax, qmax + 1, (w.d_out, w.d_in), dtype=np.int8)
    acc = hq.gemm_i32(desc, codes_dev(desc, a), codes_dev(desc, b), w.T, w.d_out)
    rows = sample_rows(w.T)
    got = to_np(acc[torch.from_numpy(rows).cuda()]).astype(np.int64)
    np.testing.assert_array_equal(got, O.int_gemm(a[rows], b))
