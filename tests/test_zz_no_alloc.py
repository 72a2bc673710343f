"""hq_quant_linear_noalloc (the static-scratch variant) against hq_quant_linear
through the C ABI: the same kernels on the same inputs, so the outputs must
be bitwise equal, on two calls in a row with the second on fewer tokens
(the scratch array keeps the first call's contents), at the largest
workspace among the workloads (square4k with per-channel centring, 26 MiB
of the 32 MiB array), and a call whose workspace would exceed the array is
refused before anything is launched."""
import dataclasses

import pytest
import torch

import hadamard_rotated_bit_amd as hq
from hadamard_rotated_bit_amd import _lib
from hadamard_rotated_bit_amd import workloads as WL
from parity import desc_for, tdev

pytestmark = pytest.mark.gpu


def setup(name, T, center=None):
    w = WL.WORKLOADS[name]
    desc = desc_for(w)
    if center is not None:
        desc = dataclasses.replace(desc, center=center)
    x = WL.gen_x(w, T=T)
    X = tdev(x, w.dtype)
    W = tdev(WL.gen_weight(w), w.dtype)
    B = torch.from_numpy(WL.gen_bias(w)).cuda()
    S = None
    if w.alpha is not None:
        S = hq.sigma(desc, hq.channel_absmax(desc, X), W, w.alpha)
    l1, l2 = WL.gen_lowrank(w)
    L1 = None if l1 is None else tdev(l1, w.dtype)
    L2 = None if l2 is None else tdev(l2, w.dtype)
    return desc, hq.prepare(desc, W, B, S, L1, L2), X


@pytest.mark.parametrize("name,T1,T2,center", [
    ("flux_proj", 1000, 300, None), ("dit_fc1", 2048, 77, None), ("lic_dh", 12288, 5, None),
    ("square4k", 8192, 1000, hq.HQ_CENTER_CHANNEL), ("tiny", 64, 1, None)])
def test_noalloc_matches_workspace_entry_point(name, T1, T2, center):
    print(f"\n[case] noalloc {name} T={T1} then {T2} center={center}", flush=True)
    desc, prep, X = setup(name, T1, center)
    assert hq.workspace_bytes(desc, T1) <= hq.NOALLOC_SCRATCH_BYTES
    for t in (T1, T2):
        Xt = X[:t].contiguous()
        ref = hq.quant_linear(desc, prep, Xt)
        got = hq.quant_linear_noalloc(desc, prep, Xt)
        torch.cuda.synchronize()
        assert torch.equal(ref, got), f"{name} T={t}"


def test_noalloc_rejects_oversize_without_launch():
    w = WL.WORKLOADS["square4k"]
    desc = desc_for(w)
    T = 12000   # codes alone: 12000 x 3072 bytes > 32 MiB
    assert hq.workspace_bytes(desc, T) > hq.NOALLOC_SCRATCH_BYTES
    X = torch.zeros(T, w.d_in, dtype=torch.bfloat16, device="cuda")
    Y = torch.full((T, w.d_out), 3.0, dtype=torch.bfloat16, device="cuda")
    prep = torch.zeros(hq.prepared_bytes(desc), dtype=torch.uint8, device="cuda")
    with pytest.raises(_lib.HqError) as e:
        hq.quant_linear_noalloc(desc, prep, X, out=Y)
    assert e.value.status == _lib.HQ_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((Y == 3.0).all())   # untouched
