"""quant_linear and quant_linear_noalloc captured in a HIP graph: every
replay must equal the eager call on the same input bitwise, with eager work
(other quant_linear calls on other buffers) run and synchronised between the
replays and the graph's input switched between two token sets. The hot path
launches kernels only (no memset or copy nodes), so the captured graph is
the same kernels with the same arguments."""
import dataclasses

import pytest
import torch

import hadamard_rotated_bit_amd as hq
from hadamard_rotated_bit_amd import workloads as WL
from parity import desc_for, tdev

pytestmark = pytest.mark.gpu


def _layer(name, gemm, T):
    w = WL.WORKLOADS[name]
    desc = dataclasses.replace(desc_for(w), gemm=gemm)
    Xa = tdev(WL.gen_x(w, T=T), w.dtype)
    Xb = tdev(WL.gen_x(w, T=T, row0=T), w.dtype)
    W = tdev(WL.gen_weight(w), w.dtype)
    S = hq.sigma(desc, hq.channel_absmax(desc, Xa), W, w.alpha) if w.alpha is not None else None
    l1, l2 = WL.gen_lowrank(w)
    prep = hq.prepare(desc, W, torch.from_numpy(WL.gen_bias(w)).cuda(), S,
                      None if l1 is None else tdev(l1, w.dtype),
                      None if l2 is None else tdev(l2, w.dtype))
    return desc, prep, Xa, Xb


@pytest.mark.parametrize("name,gemm", [("dit_fc1", hq.HQ_GEMM_AUTO), ("flux_proj", hq.HQ_GEMM_AUTO),
                                       ("flux_proj", hq.HQ_GEMM_I8)])
@pytest.mark.parametrize("noalloc", [False, True])
def test_graph_replays_match_eager(name, gemm, noalloc):
    T = 1000
    print(f"\n[case] {name} gemm={gemm} noalloc={noalloc} T={T}", flush=True)
    desc, prep, Xa, Xb = _layer(name, gemm, T)
    ws = torch.empty(hq.workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
    Ya = hq.quant_linear(desc, prep, Xa, workspace=ws)
    Yb = hq.quant_linear(desc, prep, Xb, workspace=ws)

    Xg = Xa.clone()
    out = torch.empty_like(Ya)
    wsg = torch.empty_like(ws)

    def call():
        if noalloc:
            hq.quant_linear_noalloc(desc, prep, Xg, out=out)
        else:
            hq.quant_linear(desc, prep, Xg, out=out, workspace=wsg)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    other = torch.empty_like(Ya)
    for rep in range(4):
        Xg.copy_(Xa if rep % 2 == 0 else Xb)
        g.replay()
        # eager work between the replays, on other buffers
        hq.quant_linear(desc, prep, Xb if rep % 2 == 0 else Xa, out=other, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(out, Ya if rep % 2 == 0 else Yb), f"replay {rep}"
        assert torch.equal(other, Yb if rep % 2 == 0 else Ya), f"eager call after replay {rep}"
    del g
