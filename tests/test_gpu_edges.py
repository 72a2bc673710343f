"""GPU edge cases against the oracle: empty, single and ragged token counts,
ragged output widths, degenerate rows, no / tiny / full rotation blocks, mixed
dtypes and code widths, the low-rank branch in float32, heavy outliers, and
determinism across launch configurations."""
import numpy as np
import pytest
import torch

import hadamard_rotated_bit_amd as hq
from hadamard_rotated_bit_amd import workloads as WL
from oracle import hq_oracle as O
from parity import MAX_FLIP_FRAC, XT_TOL, Y_TOL, check_codes, codes_np, rel_fro, tdev, to_np

pytestmark = pytest.mark.gpu
DT = {"f32": hq.F32, "bf16": hq.BF16}


def run_case(T, d_in, d_out, *, block, a_bits=4, w_bits=4, center=True, alpha=0.5, rank=0,
             x_dtype="f32", w_dtype="f32", y_dtype="f32", key=100, x=None, n_outliers=4,
             outlier=50.0, gemm=hq.HQ_GEMM_AUTO):
    print(f"\n[case] T={T} {d_in}->{d_out} block={block} A{a_bits}W{w_bits} center={center} "
          f"alpha={alpha} rank={rank} {x_dtype}/{w_dtype}/{y_dtype} gemm={gemm}", flush=True)
    w = WL.custom(key, T, d_in, d_out, dtype=x_dtype, block=block, alpha=alpha, center=int(center),
                  a_bits=a_bits, w_bits=w_bits, rank=rank, n_outliers=n_outliers, outlier=outlier)
    if x is None:
        x = WL.gen_x(w) if T > 0 else np.zeros((0, d_in), dtype=np.float32)
    wq = WL.Workload(**{**w.__dict__, "dtype": w_dtype})
    weight, bias = WL.gen_weight(wq), WL.gen_bias(wq)
    l1, l2 = WL.gen_lowrank(wq)
    desc = hq.Desc(d_in, d_out, block, a_bits, w_bits, center, alpha is not None, rank,
                   DT[x_dtype], DT[w_dtype], DT[y_dtype], gemm)
    sig = None
    if alpha is not None:
        sig = O.smoothing_scales(x if T > 0 else np.ones((1, d_in)), weight, alpha)
        sig = sig.astype(np.float32).astype(np.float64)
    prep = hq.prepare(desc, tdev(weight, w_dtype), torch.from_numpy(bias).cuda(),
                      None if sig is None else torch.from_numpy(sig.astype(np.float32)).cuda(),
                      None if l1 is None else tdev(l1, w_dtype),
                      None if l2 is None else tdev(l2, w_dtype))
    X = tdev(x, x_dtype)
    Y = hq.quant_linear(desc, prep, X)
    codes, s_x, mu, U = hq.act_quantize(desc, prep, X)
    ora = O.run(x, weight, bias, block=block, a_bits=a_bits, w_bits=w_bits, center=center,
                sigma=sig, l1=l1, l2=l2, out_dtype=y_dtype)
    return desc, prep, X, Y, codes, s_x, mu, U, ora


def check_all(Y, codes, s_x, ora, desc):
    err = rel_fro(to_np(Y), ora["y_out"])
    assert err <= Y_TOL, err
    ratio = np.divide(ora["xt"], ora["s_x"][:, None], out=np.zeros_like(ora["xt"]),
                      where=ora["s_x"][:, None] > 0)
    check_codes(codes_np(desc, codes, Y.shape[0]), ora["qa"], ratio, "activation codes")
    np.testing.assert_allclose(to_np(s_x), ora["s_x"], rtol=1e-5, atol=1e-30)


def test_empty_batch():
    desc, prep, X, Y, codes, s_x, mu, U, ora = run_case(0, 128, 64, block=128)
    assert Y.shape == (0, 64) and hq.code_bytes(desc, 0) == 0


ENGINES = [hq.HQ_GEMM_AUTO, hq.HQ_GEMM_I8]


@pytest.mark.parametrize("gemm", ENGINES)
@pytest.mark.parametrize("T", [1, 3, 129, 257, 1000])
def test_ragged_tokens(T, gemm):
    r = run_case(T, 256, 264, block=64, gemm=gemm)
    check_all(r[3], r[4], r[5], r[8], r[0])


@pytest.mark.parametrize("gemm", ENGINES)
@pytest.mark.parametrize("T,d_out", [(600, 1032), (700, 1160), (2100, 1536)])
def test_ragged_outputs_large_tiles(T, d_out, gemm):
    # T > 512 and d_out > 512 take the large tile shapes of both engines
    r = run_case(T, 512, d_out, block=512, gemm=gemm)
    check_all(r[3], r[4], r[5], r[8], r[0])


@pytest.mark.parametrize("gemm", ENGINES)
@pytest.mark.parametrize("rank,wd", [(0, "bf16"), (32, "bf16"), (32, "f32"), (64, "bf16")])
def test_persistent_gemm_ragged(rank, wd, gemm):
    # bf16 output with K >= 384 and M, N > 512 takes the persistent GEMM of
    # either engine: 777 tokens (three full 256-row tiles and 9 rows) by 1160
    # outputs (six 192-column tiles and 8 columns), every low-rank epilogue
    # instance (none; bf16 L2, which has no low half; fp32 L2, hi + lo; rank
    # 64, taken in 32-rank chunks)
    r = run_case(777, 1024, 1160, block=256, rank=rank, x_dtype="bf16", w_dtype=wd,
                 y_dtype="bf16", gemm=gemm)
    desc, prep, X, Y, codes, s_x, mu, U, ora = r
    check_all(Y, codes, s_x, ora, desc)
    if rank:
        err = np.linalg.norm(to_np(U) - ora["u"], axis=1) / np.linalg.norm(ora["u"], axis=1)
        assert err.max() <= 1e-4, err.max()


def test_zero_and_degenerate_rows():
    d = 128
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, d)).astype(np.float32)
    x[1] = 0.0                                   # all-zero row
    x[3] = 0.0
    x[3, 0] = 2.5                                # only channel 0: centred X~ is exactly 0
    r = run_case(6, d, 64, block=d, alpha=None, x=x)
    desc, prep, X, Y, codes, s_x, mu, U, ora = r
    c = codes_np(desc, codes, 6)
    assert not c[1].any() and not c[3].any()
    assert to_np(s_x)[1] == 0.0 and to_np(s_x)[3] == 0.0
    check_all(Y, codes, s_x, ora, desc)
    # Y of the degenerate row is b + mu c (the whole output comes from the bias correction)
    np.testing.assert_allclose(to_np(Y)[3], ora["y_full"][3], rtol=1e-5, atol=1e-6)


@pytest.mark.parametrize("block", [1, 2, 8, 32, 1024])
def test_block_sizes(block):
    r = run_case(200, 1024, 256, block=block)
    check_all(r[3], r[4], r[5], r[8], r[0])


@pytest.mark.parametrize("xd,wd,yd", [("f32", "bf16", "bf16"), ("bf16", "f32", "f32"),
                                      ("bf16", "bf16", "f32")])
def test_mixed_dtypes(xd, wd, yd):
    r = run_case(300, 384, 512, block=128, x_dtype=xd, w_dtype=wd, y_dtype=yd)
    check_all(r[3], r[4], r[5], r[8], r[0])


@pytest.mark.parametrize("ab,wb", [(8, 4), (4, 8), (8, 8)])
def test_code_widths(ab, wb):
    r = run_case(300, 256, 256, block=256, a_bits=ab, w_bits=wb)
    check_all(r[3], r[4], r[5], r[8], r[0])
    assert np.abs(codes_np(r[0], r[4], 300)).max() <= 2 ** (ab - 1) - 1


@pytest.mark.parametrize("gemm", ENGINES)
@pytest.mark.parametrize("rank,xd", [(16, "f32"), (48, "bf16"), (64, "f32")])
def test_low_rank(rank, xd, gemm):
    r = run_case(260, 512, 384, block=256, rank=rank, x_dtype=xd, w_dtype=xd, y_dtype=xd,
                 gemm=gemm)
    desc, prep, X, Y, codes, s_x, mu, U, ora = r
    check_all(Y, codes, s_x, ora, desc)
    err = np.linalg.norm(to_np(U) - ora["u"], axis=1) / np.linalg.norm(ora["u"], axis=1)
    assert err.max() <= 1e-4, err.max()


@pytest.mark.parametrize("T,d_in,rank,xd", [(130, 2048, 32, "bf16"), (300, 3072, 32, "bf16"),
                                         (77, 1152, 16, "f32"), (129, 1024, 64, "f32"),
                                         (1, 512, 48, "bf16"), (200, 1024, 16, "bf16"),
                                         (4200, 3072, 32, "bf16"), (4500, 3072, 16, "f32")])
def test_low_rank_split_matches_one_pass(T, d_in, rank, xd):
    # quant_linear forms U in two passes over slices of d_in (workspace for the
    # slice products); act_quantize has no workspace and runs the one-pass
    # kernel. The slices are the one-pass kernel's wave partition summed in
    # the same order, so U and therefore Y are bit-identical. The slice count
    # follows the row count: 8 slices of 384 channels for d_in 3072 at 300
    # rows, 6 of 512 at 4200 and 4500 rows (33-36 blocks of 128 rows, so 6
    # slices fill the compute units in one round and 8 would not).
    r = run_case(T, d_in, 264, block=128, rank=rank, x_dtype=xd, w_dtype=xd, y_dtype=xd)
    desc, prep, X, Y, codes, s_x, mu, U, ora = r
    check_all(Y, codes, s_x, ora, desc)
    err = np.linalg.norm(to_np(U) - ora["u"], axis=1) / np.linalg.norm(ora["u"], axis=1)
    assert err.max() <= 1e-4, err.max()
    assert torch.equal(Y, hq.gemm_dequant(desc, prep, codes, s_x, mu, U))
    # the stage entry point with a workspace runs the two-pass form itself:
    # the same bits as the one-pass stage
    ws = torch.empty(hq.workspace_bytes(desc, T), dtype=torch.uint8, device=X.device)
    c2, s2, m2, U2 = hq.act_quantize(desc, prep, X, workspace=ws)
    np.testing.assert_array_equal(codes_np(desc, c2, T), codes_np(desc, codes, T))
    assert torch.equal(s2, s_x) and torch.equal(m2, mu) and torch.equal(U2, U)
    small = torch.empty(hq.workspace_bytes(desc, T) - 256, dtype=torch.uint8, device=X.device)
    with pytest.raises(hq.HqError):
        hq.act_quantize(desc, prep, X, workspace=small)


@pytest.mark.parametrize("T,d_in,block,rank,alpha,center,bits,gemm", [
    (300, 3072, 1024, 32, 0.5, True, 4, hq.HQ_GEMM_AUTO),
    (1, 3072, 512, 16, 0.5, True, 4, hq.HQ_GEMM_AUTO),
    (17, 2560, 512, 32, None, False, 4, hq.HQ_GEMM_AUTO),
    (64, 2560, 512, 16, 0.5, True, 4, hq.HQ_GEMM_AUTO),
    (4100, 3072, 1024, 32, None, True, 4, hq.HQ_GEMM_AUTO),
    (300, 3072, 1024, 32, 0.5, True, 4, hq.HQ_GEMM_I8),
    (129, 2560, 512, 16, 0.5, True, 8, hq.HQ_GEMM_AUTO)])
def test_low_rank_wide_rows(T, d_in, block, rank, alpha, center, bits, gemm):
    # bf16 input with d_in 2560 or 3072 (64 lanes per row in the row kernel),
    # blocks of >= 512 channels and rank 16 or 32, with and without smoothing
    # and centring: the flux_proj geometry at ragged row counts (1, 17, 300,
    # 4100 rows: partial 64-row projection blocks and 8-row transform
    # blocks). These geometries run the row transform and the down
    # projection in one launch through every entry point (quant_linear,
    # act_quantize with and without a workspace), so U, and therefore Y, are
    # the same bits through all three. The int8 engine and 8-bit codes take
    # the transform role's int8 code writer.
    r = run_case(T, d_in, 520, block=block, rank=rank, alpha=alpha, center=center,
                 a_bits=bits, w_bits=bits, x_dtype="bf16", w_dtype="bf16", y_dtype="bf16",
                 gemm=gemm)
    desc, prep, X, Y, codes, s_x, mu, U, ora = r
    check_all(Y, codes, s_x, ora, desc)
    err = np.linalg.norm(to_np(U) - ora["u"], axis=1) / np.linalg.norm(ora["u"], axis=1)
    print(f"U: max row error {err.max():.2e}")
    assert err.max() <= 1e-4, err.max()
    rms = np.sqrt(np.mean(ora["y"] ** 2, axis=1))
    assert np.all(np.abs(to_np(mu) - ora["mu"]) <= XT_TOL * rms)
    assert torch.equal(Y, hq.gemm_dequant(desc, prep, codes, s_x, mu, U))
    ws = torch.empty(hq.workspace_bytes(desc, T), dtype=torch.uint8, device=X.device)
    c2, s2, m2, U2 = hq.act_quantize(desc, prep, X, workspace=ws)
    np.testing.assert_array_equal(codes_np(desc, c2, T), codes_np(desc, codes, T))
    assert torch.equal(s2, s_x) and torch.equal(m2, mu) and torch.equal(U2, U)


def test_one_launch_activation_matches_separate_kernels():
    # The same bf16 values given as bf16 X (the one-launch activation kernel)
    # and as float32 X (the row kernel, then the two-pass down projection):
    # the transforms run the same float32 arithmetic, so codes, scales and
    # means are bit-identical; U is summed in a different order and agrees to
    # float32 rounding.
    T, d_in, d_out, rank = 300, 3072, 520, 32
    print(f"\n[case] one launch vs separate kernels T={T} {d_in}->{d_out} rank={rank}", flush=True)
    w = WL.custom(321, T, d_in, d_out, dtype="bf16", block=1024, alpha=0.5, center=1, rank=rank)
    x, weight, bias = WL.gen_x(w), WL.gen_weight(w), WL.gen_bias(w)
    l1, l2 = WL.gen_lowrank(w)
    sig = torch.from_numpy(O.smoothing_scales(x, weight, 0.5).astype(np.float32)).cuda()
    xb = tdev(x, "bf16")
    outs = []
    for xd, X in ((hq.BF16, xb), (hq.F32, xb.float())):
        desc = hq.Desc(d_in, d_out, 1024, 4, 4, True, True, rank, xd, hq.BF16, hq.BF16)
        prep = hq.prepare(desc, tdev(weight, "bf16"), torch.from_numpy(bias).cuda(), sig,
                          tdev(l1, "bf16"), tdev(l2, "bf16"))
        ws = torch.empty(hq.workspace_bytes(desc, T), dtype=torch.uint8, device="cuda")
        c, s_x, mu, U = hq.act_quantize(desc, prep, X, workspace=ws)
        outs.append((codes_np(desc, c, T), s_x, mu, U))
    (cb, sb, mb, ub), (cf, sf, mf, uf) = outs
    np.testing.assert_array_equal(cb, cf)
    assert torch.equal(sb, sf) and torch.equal(mb, mf)
    err = (torch.linalg.norm(ub - uf, dim=1) / torch.linalg.norm(uf, dim=1)).max().item()
    print(f"U: largest row difference {err:.2e}")
    assert err <= 1e-6, err


def test_heavy_outliers_and_no_centring():
    r = run_case(400, 2048, 512, block=2048, center=False, alpha=None, n_outliers=16,
                 outlier=1000.0)
    check_all(r[3], r[4], r[5], r[8], r[0])
    assert not to_np(r[6]).any()        # mu is zero without centring


def test_deterministic_across_launch_configs():
    # the same 300 tokens inside a 2048-token batch (different GEMM tiling)
    # give bit-identical accumulators and outputs
    w = WL.custom(300, 2048, 1024, 768, dtype="bf16", block=256, alpha=None)
    x = WL.gen_x(w)
    desc = hq.Desc(1024, 768, 256, 4, 4, True, False, 0, hq.BF16, hq.BF16, hq.BF16)
    prep = hq.prepare(desc, tdev(WL.gen_weight(w), "bf16"), torch.from_numpy(WL.gen_bias(w)).cuda())
    Xb = tdev(x, "bf16")
    Yb = hq.quant_linear(desc, prep, Xb)
    Ys = hq.quant_linear(desc, prep, Xb[:300].contiguous())
    assert torch.equal(Yb[:300], Ys)
    assert torch.equal(Yb, hq.quant_linear(desc, prep, Xb))
    v = hq.prepared_views(desc, prep)
    codes = hq.act_quantize(desc, prep, Xb)[0]
    a1 = hq.gemm_i32(desc, codes, v["w_codes"], 2048, 768)
    a2 = hq.gemm_i32(desc, codes[:hq.code_bytes(desc, 300)].clone(), v["w_codes"], 300, 768)
    assert torch.equal(a1[:300], a2)


def test_check_prepared_header():
    w = WL.custom(301, 16, 256, 128, block=128)
    desc = hq.Desc(256, 128, 128, 4, 4, True, False, 0)
    prep = hq.prepare(desc, tdev(WL.gen_weight(w), "f32"))
    hq.check_prepared(desc, prep)
    other = hq.Desc(256, 128, 64, 4, 4, True, False, 0)
    with pytest.raises(hq.HqError):
        hq.check_prepared(other, prep)
