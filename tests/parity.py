"""Shared helpers for the GPU parity tests: build a case, run the oracle, compare.

Tolerances (fixed here, applied by every GPU test):
* sigma: relative error <= 1e-6.
* float transform X~ (and mu): per-row ||dX~|| / ||X~|| <= 1e-5, |dmu| <= 1e-5 rms(y).
* integer codes: equal except that at most 1e-4 of the elements may differ by
  exactly one code, and each such element must be a rounding near-tie in the
  oracle: |frac(|v|) - 1/2| <= tie_window(qmax) with v = x~ / s in float64.
  The oracle decides round(v / s) in float64 (HaTQ Eq. (3) as written); the
  kernel decides the same quotient from its float32 transform, so a flip
  needs the two to straddle a half-integer. The window bounds that float32
  error: v / s = qmax v / max|v|, and the kernel's value carries the relative
  error of its transform (a sum of L <= 13 butterfly stages, each adding a
  rounding of u = 2^-24 relative to its partial sums, which in quadrature
  gives ~sqrt(L / 3) u relative to the output rms, below 6 standard
  deviations times 2 u of max|v| over ~10^8 elements), of the channel scaling
  and centring (one rounding each), of max|v| (the same error) and of the
  float32 reciprocal qmax / max|v| (u): about 16 u relative in all, i.e.
  |delta(v / s)| <= 16 u qmax. The window takes 8 times that, qmax 2^-17
  (5.3e-5 for 4-bit, 9.7e-4 for 8-bit codes).
* int32 accumulators: bit-exact when the GEMM is fed the oracle's codes.
* output: ||Y_gpu - Y_oracle||_F / ||Y_oracle||_F <= 1e-3, same output dtype.
"""
from __future__ import annotations

import functools

import numpy as np
import torch

from oracle import hq_oracle as O
from hadamard_rotated_bit_amd import workloads as WL
import hadamard_rotated_bit_amd as hq
import codefmt

MAX_FLIP_FRAC = 1e-4


def tie_window(qmax: int) -> float:
    """Largest distance of a flipped code's oracle quotient from a half-integer
    (see the module docstring)."""
    return float(qmax) * 2.0 ** -17
Y_TOL = 1e-3
XT_TOL = 1e-5


def desc_for(w: WL.Workload, gemm: int = hq.HQ_GEMM_AUTO) -> hq.Desc:
    dt = hq.BF16 if w.dtype == "bf16" else hq.F32
    return hq.Desc(w.d_in, w.d_out, w.block, w.a_bits, w.w_bits, int(w.center),
                   w.alpha is not None, w.rank, dt, dt, dt, gemm, w.group)


# (workload, GEMM engine) pairs the parity tests run: every workload on the
# automatic engine, and the 4-bit ones also on the int8 engine.
ENGINE_CASES = [(n, hq.HQ_GEMM_AUTO) for n in WL.PARITY_ORDER] + [
    (n, hq.HQ_GEMM_I8) for n in WL.PARITY_ORDER
    if WL.WORKLOADS[n].a_bits == 4 and WL.WORKLOADS[n].w_bits == 4]


def case_id(c) -> str:
    return f"{c[0]}-{'i8' if c[1] == hq.HQ_GEMM_I8 else 'auto'}"


def tdev(a: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    return t.cuda()


class Case:
    """Inputs of a workload (first T rows), the oracle's results, the GPU prepared blob."""

    def __init__(self, w: WL.Workload, T: int, x=None, gemm: int = hq.HQ_GEMM_AUTO):
        self.w = w
        self.T = T
        self.desc = desc_for(w, gemm)
        self.x = WL.gen_x(w, T=T) if x is None else x
        self.weight = WL.gen_weight(w)
        self.bias = WL.gen_bias(w)
        self.l1, self.l2 = WL.gen_lowrank(w)
        if w.alpha is not None:
            self.sigma64 = O.smoothing_scales(self.x, self.weight, w.alpha)
            self.sigma32 = self.sigma64.astype(np.float32)
        else:
            self.sigma64 = None
            self.sigma32 = None
        sig = None if self.sigma32 is None else self.sigma32.astype(np.float64)
        self.ora = O.run(self.x, self.weight, self.bias, block=w.block, a_bits=w.a_bits,
                         w_bits=w.w_bits, center=int(w.center), sigma=sig, l1=self.l1,
                         l2=self.l2, out_dtype=w.out_dtype, group=w.group)
        # device tensors
        self.X = tdev(self.x, w.dtype)
        self.W = tdev(self.weight, w.dtype)
        self.B = torch.from_numpy(self.bias).cuda()
        self.S = None if self.sigma32 is None else torch.from_numpy(self.sigma32).cuda()
        self.L1 = None if self.l1 is None else tdev(self.l1, w.dtype)
        self.L2 = None if self.l2 is None else tdev(self.l2, w.dtype)
        self.prep = hq.prepare(self.desc, self.W, self.B, self.S, self.L1, self.L2)


@functools.lru_cache(maxsize=None)
def small_case(name: str, T: int = 300, gemm: int = hq.HQ_GEMM_AUTO) -> Case:
    print(f"\n[case] {name} T={T} gemm={gemm}", flush=True)
    return Case(WL.WORKLOADS[name], T, gemm=gemm)


def check_codes(gpu_codes, ora_codes, ora_v, what: str):
    """Tie-aware code comparison (see module docstring)."""
    g = np.asarray(gpu_codes, dtype=np.int64)
    o = np.asarray(ora_codes, dtype=np.int64)
    assert g.shape == o.shape, (g.shape, o.shape)
    d = g - o
    assert np.abs(d).max(initial=0) <= 1, f"{what}: a code differs by more than 1"
    bad = d != 0
    frac = bad.mean() if bad.size else 0.0
    assert frac <= MAX_FLIP_FRAC, f"{what}: {bad.sum()} flipped codes ({frac:.2e})"
    if bad.any():
        # the row maximum codes to +-qmax, so the largest oracle code is qmax
        qmax = int(np.abs(o).max())
        av = np.abs(np.asarray(ora_v)[bad])
        dist = np.abs(av - np.floor(av) - 0.5)
        win = tie_window(qmax)
        print(f"{what}: {int(bad.sum())} flipped code(s), largest distance from a tie "
              f"{dist.max():.2e} (window {win:.2e})", flush=True)
        assert dist.max() <= win, f"{what}: flip not at a tie (distance {dist.max():.3e})"
    return int(bad.sum())


def codes_np(desc: hq.Desc, buf: torch.Tensor, rows: int, idx=None) -> np.ndarray:
    """Integer codes [rows, d_in] (or rows `idx`) of a device code buffer of
    `rows` rows, read on the host from the format's definition (codefmt.py)."""
    fmt = codefmt.fmt_of(desc.a_bits, desc.w_bits, desc.gemm)
    assert hq.code_format(desc) == fmt
    assert hq.code_bytes(desc, rows) == codefmt.nbytes(fmt, rows, desc.d_in)
    return codefmt.decode(fmt, buf.detach().cpu().numpy(), rows, desc.d_in, idx)


def codes_dev(desc: hq.Desc, codes: np.ndarray) -> torch.Tensor:
    """Device code buffer holding integer codes [rows, d_in]."""
    fmt = codefmt.fmt_of(desc.a_bits, desc.w_bits, desc.gemm)
    return torch.from_numpy(codefmt.encode(fmt, codes)).cuda()


def rel_fro(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def to_np(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        t = t.float()
    return t.detach().cpu().numpy()
