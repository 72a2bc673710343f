"""The GEMM engines behind hq_gemm_dequant, held bit-exact through the bf16
output path (the launch configuration quant_linear uses for bf16 outputs and
K >= 384: on the FP6 engine the persistent kernel, which walks several tiles
per block).

With unit scales (s_x = s_w = 1), c = 0, b = 0 and mu = 0 the epilogue of
HaTQ Eq. (18) reduces to Y = acc. Sparse activation codes (at most five
nonzero codes of magnitude <= 7 per row against weight codes of magnitude
<= 7) keep |acc| <= 245 < 256, where every integer is exactly a bf16 value,
so Y must equal the oracle's integer product exactly. T = 8000 is not a
multiple of the 256-row tile (a ragged last row tile) and gives more tiles
than the chip has compute units.
"""
import numpy as np
import pytest
import torch

import hadamard_rotated_bit_amd as hq
from oracle import hq_oracle as O
from parity import codes_dev, tdev, to_np

pytestmark = pytest.mark.gpu


def sparse_codes(rng, rows, d, nnz, qmax):
    a = np.zeros((rows, d), dtype=np.int64)
    for r in range(rows):
        k = rng.choice(d, size=nnz, replace=False)
        a[r, k] = rng.integers(1, qmax + 1, nnz) * rng.choice([-1, 1], nnz)
    return a


@pytest.mark.parametrize("gemm", [hq.HQ_GEMM_AUTO, hq.HQ_GEMM_I8], ids=["fp6", "i8"])
@pytest.mark.parametrize("rank", [0, 32])
def test_gemm_dequant_equals_accumulators(gemm, rank):
    T, d_in, d_out = 8000, 1152, 4608
    print(f"\n[case] exact GEMM through the bf16 epilogue T={T} {d_in}->{d_out} "
          f"gemm={gemm} rank={rank}", flush=True)
    desc = hq.Desc(d_in, d_out, 128, 4, 4, hq.HQ_CENTER_TOKEN, False, rank,
                   hq.BF16, hq.BF16, hq.BF16, gemm)
    rng = np.random.default_rng(4242 + rank + 7 * gemm)
    a = sparse_codes(rng, T, d_in, 5, 7)
    b = rng.integers(-7, 8, (d_out, d_in))
    weight = tdev(rng.standard_normal((d_out, d_in)) * 0.02, "bf16")
    L1 = L2 = None
    if rank:
        L1 = tdev(rng.standard_normal((d_in, rank)) * 0.02, "bf16")
        L2 = tdev(rng.standard_normal((rank, d_out)) * 0.02, "bf16")
    prep = hq.prepare(desc, weight, None, None, L1, L2)
    # unit weight scales, c = 0, b = 0 and the test's weight codes in the blob
    v = hq.prepared_views(desc, prep)
    v["s_w"].fill_(1.0)
    v["c"].zero_()
    v["bias"].zero_()
    wc = codes_dev(desc, b)
    L = hq.layout(desc)
    prep[L.w_codes:L.w_codes + wc.numel()].copy_(wc)
    codes = codes_dev(desc, a)
    s_x = torch.ones(T, dtype=torch.float32, device="cuda")
    mu = torch.zeros(T, dtype=torch.float32, device="cuda")
    U = torch.zeros(T, rank, dtype=torch.float32, device="cuda") if rank else None
    for t_ in (T, 300):   # two calls in a row, the second on a prefix
        Y = hq.gemm_dequant(desc, prep, codes, s_x[:t_].contiguous(), mu[:t_].contiguous(),
                            None if U is None else U[:t_].contiguous())
        torch.cuda.synchronize()
        acc = O.int_gemm(a[:t_], b)
        assert np.abs(acc).max() <= 256
        np.testing.assert_array_equal(to_np(Y).astype(np.int64), acc)
