"""GPU parity of group-wise scales (descriptor group = 64; data-free int4 blog,
"Hadamard rotation: the int4 improvement": one scale per row and group of 64
input channels, one 64-point Hadamard block per group) against the CPU oracle.

Cases: the flux_g64 workload (FLUX-scale 3072 -> 12288 projection, rank 32)
on its first 300 tokens under each centring mode; ragged shapes (token
counts off the 128-row tile and the 4-row code group, output widths off the
128-column tile, one 128-channel stage, f32 output); the GEMM alone fed the
oracle's own codes and scales; zero rows; and flux_g64 at its full 4608
tokens on sampled rows. Tolerances are those of tests/parity.py; the GEMM
fed the oracle's codes is held to float32 summation accuracy.
"""
import dataclasses

import numpy as np
import pytest
import torch

import hadamard_rotated_bit_amd as hq
from hadamard_rotated_bit_amd import workloads as WL
from oracle import hq_oracle as O
from parity import (Y_TOL, Case, check_codes, codes_dev, codes_np, desc_for, rel_fro, tdev,
                    to_np)

pytestmark = pytest.mark.gpu
GROUP = 64
_CASES = {}


def group_case(name: str, T: int = 300, center=None) -> Case:
    key = (name, T, center)
    if key not in _CASES:
        w = WL.WORKLOADS[name]
        if center is not None:
            w = dataclasses.replace(w, center=center)
        print(f"\n[case] group-wise {name} T={T} center={w.center}", flush=True)
        _CASES[key] = Case(w, T)
    return _CASES[key]


def ratio_of(xt, s):
    """x~ / s per element, s [rows, groups] repeated over each group's channels."""
    sr = np.repeat(s, GROUP, axis=1)
    return np.divide(xt, sr, out=np.zeros_like(xt), where=sr > 0)


def check_case(c: Case):
    o, d = c.ora, c.desc
    G = d.d_in // GROUP
    # weights: codes and per-(channel, group) scales of the prepared blob
    v = hq.prepared_views(d, c.prep)
    assert tuple(v["s_w"].shape) == (G, d.d_out)
    np.testing.assert_allclose(to_np(v["s_w"]).T, o["s_w"], rtol=1e-5, atol=1e-30)
    check_codes(codes_np(d, v["w_codes"], d.d_out), o["qw"], ratio_of(o["wt"], o["s_w"]),
                "weight codes")
    if int(c.w.center) == O.CENTER_CHANNEL:   # the correction is the per-call bias instead
        assert not to_np(v["c"]).any()
    else:
        np.testing.assert_allclose(to_np(v["c"]), o["c"], rtol=1e-4,
                                   atol=1e-5 * np.abs(o["wt"]).sum(axis=1).max())
    # activations
    codes, s_x, mu, U = hq.act_quantize(d, c.prep, c.X)
    assert tuple(s_x.shape) == (G, c.T)
    flips = check_codes(codes_np(d, codes, c.T), o["qa"], ratio_of(o["xt"], o["s_x"]),
                        "activation codes")
    np.testing.assert_allclose(to_np(s_x).T, o["s_x"], rtol=1e-5, atol=1e-30)
    # output, and the staged path gives the same bits
    Y = hq.quant_linear(d, c.prep, c.X)
    err = rel_fro(to_np(Y), o["y_out"])
    print(f"{c.w.name} center={c.w.center}: {flips} flipped codes, rel Frobenius error {err:.3e}")
    assert err <= Y_TOL, err
    if int(c.w.center) == O.CENTER_CHANNEL:
        _, bias_eff = hq.channel_center(d, c.prep, c.X)
        Y2 = hq.gemm_dequant(d, c.prep, codes, s_x, bias_eff, U)
    else:
        Y2 = hq.gemm_dequant(d, c.prep, codes, s_x, mu, U)
    assert torch.equal(Y, Y2)


@pytest.mark.parametrize("center", [O.CENTER_NONE, O.CENTER_TOKEN, O.CENTER_CHANNEL])
def test_group_flux(center):
    check_case(group_case("flux_g64", 300, center))


@pytest.mark.parametrize("T,d_in,d_out,block,rank,dtype", [
    (1, 128, 128, 64, 0, "f32"),       # one stage, one token
    (77, 128, 136, 64, 0, "f32"),      # ragged tokens and output columns
    (131, 256, 264, 32, 16, "bf16"),   # block smaller than the group, rank 16
    (300, 1152, 520, 128, 32, "bf16"), # block larger than the group
    (257, 384, 1000, 64, 0, "f32"),    # odd stage count, ragged column tile
])
def test_group_ragged(T, d_in, d_out, block, rank, dtype):
    w = WL.custom(400 + T, T, d_in, d_out, dtype=dtype, block=block, alpha=None, center=1,
                  rank=rank, n_outliers=2, group=GROUP)
    check_case(Case(w, T))


def test_group_gemm_on_oracle_codes():
    # the GEMM and epilogue alone: fed the oracle's codes and float32 scales,
    # the output equals the oracle's per-group scaled sum to float32 accuracy
    # (f32 output; the group products are exact integers on both sides)
    w = WL.custom(450, 200, 512, 392, dtype="f32", block=64, alpha=None, center=1, rank=0,
                  n_outliers=3, group=GROUP)
    c = Case(w, 200)
    o, d = c.ora, c.desc
    sx32 = o["s_x"].astype(np.float32)
    sw32 = o["s_w"].astype(np.float32)
    mu32 = o["mu"].astype(np.float32)
    L = hq.layout(d)
    G = d.d_in // GROUP
    # overwrite the blob's weight codes and scales with the oracle's
    sw_dev = torch.zeros(G, L.d_out_pad, dtype=torch.float32)
    sw_dev[:, :d.d_out] = torch.from_numpy(np.ascontiguousarray(sw32.T))
    c.prep[L.w_scale:L.w_scale + 4 * G * L.d_out_pad].copy_(sw_dev.view(torch.uint8).view(-1).cuda())
    wc = codes_dev(d, o["qw"])
    c.prep[L.w_codes:L.w_codes + wc.numel()].copy_(wc)
    codes = codes_dev(d, o["qa"])
    s_x = torch.from_numpy(np.ascontiguousarray(sx32.T)).cuda()
    Y = to_np(hq.gemm_dequant(d, c.prep, codes, s_x, torch.from_numpy(mu32).cuda()))
    acc = O.group_product(o["qa"], sx32.astype(np.float64), o["qw"], sw32.astype(np.float64),
                          GROUP)
    ref = acc + c.bias[None, :] + mu32.astype(np.float64)[:, None] * to_np(
        hq.prepared_views(d, c.prep)["c"]).astype(np.float64)[None, :]
    scale = np.abs(O.group_product(np.abs(o["qa"]), sx32.astype(np.float64), np.abs(o["qw"]),
                                   sw32.astype(np.float64), GROUP)) + np.abs(ref)
    assert np.all(np.abs(Y - ref) <= 1e-5 * scale + 1e-30)


def test_group_zero_rows():
    # rows of zeros: every group scale is 0, codes are 0, Y = b (+ the
    # low-rank term of a zero input, also 0)
    w = WL.WORKLOADS["flux_g64"]
    x = WL.gen_x(w, T=12)
    x[[0, 5, 11]] = 0.0
    c = Case(w, 12, x=x)
    codes, s_x, _, _ = hq.act_quantize(c.desc, c.prep, c.X)
    s = to_np(s_x)
    assert not s[:, [0, 5, 11]].any() and s[:, [1, 2, 3]].all()
    q = codes_np(c.desc, codes, 12)
    assert not q[[0, 5, 11]].any()
    Y = to_np(hq.quant_linear(c.desc, c.prep, c.X))
    ref = O.round_to_dtype(np.broadcast_to(c.bias, (3, w.d_out)), w.out_dtype)
    assert np.array_equal(Y[[0, 5, 11]], ref)
    assert rel_fro(Y, c.ora["y_out"]) <= Y_TOL


def test_group_full_size_sampled():
    # flux_g64 at its full 4608 tokens (the launch the benchmark times): 64
    # sampled tokens against the oracle's steps on those rows (rows are
    # independent without per-channel centring)
    w = WL.WORKLOADS["flux_g64"]
    print(f"\n[case] group-wise full-size flux_g64 T={w.T}", flush=True)
    desc = desc_for(w)
    x = WL.gen_x(w)
    weight, bias = WL.gen_weight(w), WL.gen_bias(w)
    l1, l2 = WL.gen_lowrank(w)
    X = tdev(x, w.dtype)
    prep = hq.prepare(desc, tdev(weight, w.dtype), torch.from_numpy(bias).cuda(), None,
                      tdev(l1, w.dtype), tdev(l2, w.dtype))
    Y = hq.quant_linear(desc, prep, X)
    torch.cuda.synchronize()
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([np.arange(8), rng.choice(np.arange(8, w.T - 8), 48,
                                                              replace=False),
                                     np.arange(w.T - 8, w.T)]))
    y_s = to_np(Y[torch.from_numpy(rows).cuda()])
    del Y, X
    o = O.run(x[rows], weight, bias, block=w.block, a_bits=w.a_bits, w_bits=w.w_bits,
              center=int(w.center), l1=l1, l2=l2, out_dtype=w.out_dtype, group=w.group)
    err = rel_fro(y_s, o["y_out"])
    print(f"flux_g64 full size: sampled rel Frobenius error {err:.3e}")
    assert err <= Y_TOL, err
