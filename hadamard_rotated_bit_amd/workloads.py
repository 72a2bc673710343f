"""Seeded synthetic workloads for the rotated-and-centred quantised linear layer.

This module only draws numbers and names shapes. It contains none of the
layer's arithmetic (no scaling, rotation, centring or quantisation), so the
GPU path and the CPU oracle can both consume its arrays without sharing any
of the method's code.

Every array comes from numpy's counter-based Philox generator keyed by
``seed = 1_000_003 * k + stream`` (k = workload id, stream = which tensor),
so a workload is reproducible bit-for-bit on any host with this numpy.
bf16 tensors are drawn in fp32 and rounded once to bf16 (round to nearest,
ties to even); they are returned as float32 arrays holding bf16-representable
values together with the dtype tag, so both paths read identical bytes.

The five named workloads stand in for the pages' models and data, which are
not available here:

* ``tiny``      -- 64 x 128 -> 256 fp32 toy layer, full 128-point rotation,
                   four outlier channels x50 (HadaNorm W4A4 setting).
* ``dit_fc1``   -- 8192 x 1152 -> 4608 bf16, a PixArt-Sigma-like DiT MLP fc1
                   over two 4096-token images; 1 % outlier channels scaled
                   log-uniformly in [20, 100]; block-diagonal 128-point rotation.
* ``square4k``  -- 8192 x 4096 -> 4096 bf16, Student-t(3) activations plus
                   per-channel means ~ N(0, 2^2); one 4096-point rotation;
                   run with and without centring (``square4k_nc`` is the
                   same layer and the same numbers with centring off).
* ``lic_dh``    -- 12288 x 256 -> 256 fp32, a learned-image-coding 1x1 conv
                   (8 latents of 32 x 48 positions, channels last, token
                   index (n*32 + h)*48 + w); Laplace(0,1) with 8 channels x30;
                   double-Hadamard W8A8 (no smoothing, no centring).
* ``flux_proj`` -- 4608 x 3072 -> 12288 bf16, a FLUX-scale joint-attention
                   projection (4096 image + 512 text tokens); 0.5 % outlier
                   channels x50; three 1024-point blocks; rank-32 bf16
                   low-rank branch.

Two more workloads exercise the next rows (not among the five above):

* ``flux_g64``  -- flux_proj's shape and value distribution with the data-free
                   int4 blog's recipe: 64-point Hadamard blocks, one scale per
                   row and 64-channel group, rank-32 branch, no smoothing, no
                   centring.
* ``lic_wh``    -- lic_dh's shape and value distribution as a weight-only
                   Hadamard layer with integer requantisation: int8 input
                   codes with one per-tensor scale, H_256 on the output
                   channels, int8 output codes.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np

# Stream ids (the second half of the Philox key).
S_X, S_W, S_B, S_OUT_IDX, S_OUT_FAC, S_CH_MEAN, S_L1, S_L2 = range(8)


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and options of one layer workload (no arithmetic)."""
    key: int               # workload id used in the seed
    name: str
    T: int                 # tokens
    d_in: int
    d_out: int
    dtype: str             # "f32" or "bf16": X, weight, L1, L2 and Y dtype
    block: int             # Hadamard block size (power of two dividing d_in)
    alpha: Optional[float]  # smoothing exponent; None means sigma == 1
    center: int            # 1: per-token mean centring on
    a_bits: int
    w_bits: int
    rank: int              # low-rank branch rank (0 = none)
    x_dist: str            # "normal", "student_t3_means", "laplace"
    n_outliers: int        # number of outlier channels in X
    outlier_lo: float      # outlier factor range (log-uniform); lo == hi = fixed
    outlier_hi: float
    w_std: float
    b_std: float = 0.01
    lr_std: float = 0.02
    mean_std: float = 0.0  # per-channel mean std (student_t3_means only)
    group: int = 0         # 0: one scale per row; 64: one per row and 64-channel group

    @property
    def out_dtype(self) -> str:
        return self.dtype


WORKLOADS = {
    "tiny": Workload(1, "tiny", 64, 128, 256, "f32", 128, 0.5, 1, 4, 4, 0,
                     "normal", 4, 50.0, 50.0, 0.02),
    "dit_fc1": Workload(2, "dit_fc1", 8192, 1152, 4608, "bf16", 128, 0.5, 1, 4, 4, 0,
                        "normal", 12, 20.0, 100.0, 0.02),
    "square4k": Workload(3, "square4k", 8192, 4096, 4096, "bf16", 4096, None, 1, 4, 4, 0,
                         "student_t3_means", 0, 1.0, 1.0, 0.015, mean_std=2.0),
    # the same workload id (so the same X, weight and bias) with centring off
    "square4k_nc": Workload(3, "square4k_nc", 8192, 4096, 4096, "bf16", 4096, None, 0, 4, 4, 0,
                            "student_t3_means", 0, 1.0, 1.0, 0.015, mean_std=2.0),
    "lic_dh": Workload(4, "lic_dh", 12288, 256, 256, "f32", 256, None, 0, 8, 8, 0,
                       "laplace", 8, 30.0, 30.0, 0.05),
    "flux_proj": Workload(5, "flux_proj", 4608, 3072, 12288, "bf16", 1024, 0.5, 1, 4, 4, 32,
                          "normal", 15, 50.0, 50.0, 0.02),
    "flux_g64": Workload(6, "flux_g64", 4608, 3072, 12288, "bf16", 64, None, 0, 4, 4, 32,
                         "normal", 15, 50.0, 50.0, 0.02, group=64),
    "lic_wh": Workload(7, "lic_wh", 12288, 256, 256, "f32", 256, None, 0, 8, 8, 0,
                       "laplace", 8, 30.0, 30.0, 0.05),
}
ORDER = ["tiny", "dit_fc1", "square4k", "lic_dh", "flux_proj"]
# the five plus the square projection's second run (centring off)
PARITY_ORDER = ORDER[:3] + ["square4k_nc"] + ORDER[3:]
GROUP_ORDER = ["flux_g64"]
WH_ORDER = ["lic_wh"]


def rng(key: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=1_000_003 * key + stream))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> nearest bf16 (ties to even), returned as float32 values."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    u = ((u + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return u.view(np.float32)


def _cast(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.asarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def gen_x(w: Workload, T: Optional[int] = None, row0: int = 0) -> np.ndarray:
    """Activations [T, d_in] for workload ``w`` (rows row0 .. row0+T-1).

    Rows are drawn from one stream in order, so any row range is a slice of
    the full workload's X.
    """
    T = w.T if T is None else T
    g = rng(w.key, S_X)
    n_skip = row0 * w.d_in
    if w.x_dist == "normal":
        if n_skip:
            g.standard_normal(n_skip, dtype=np.float64)
        x = g.standard_normal((T, w.d_in))
    elif w.x_dist == "laplace":
        if n_skip:
            g.laplace(0.0, 1.0, n_skip)
        x = g.laplace(0.0, 1.0, (T, w.d_in))
    elif w.x_dist == "student_t3_means":
        if n_skip:
            g.standard_t(3.0, n_skip)
        x = g.standard_t(3.0, (T, w.d_in))
        means = rng(w.key, S_CH_MEAN).normal(0.0, w.mean_std, w.d_in)
        x = x + means[None, :]
    else:
        raise ValueError(w.x_dist)
    if w.n_outliers:
        idx = rng(w.key, S_OUT_IDX).choice(w.d_in, size=w.n_outliers, replace=False)
        if w.outlier_lo == w.outlier_hi:
            fac = np.full(w.n_outliers, w.outlier_lo)
        else:
            fac = np.exp(rng(w.key, S_OUT_FAC).uniform(np.log(w.outlier_lo),
                                                       np.log(w.outlier_hi), w.n_outliers))
        x[:, idx] *= fac[None, :]
    return _cast(x, w.dtype)


def outlier_channels(w: Workload) -> np.ndarray:
    if not w.n_outliers:
        return np.zeros(0, dtype=np.int64)
    return rng(w.key, S_OUT_IDX).choice(w.d_in, size=w.n_outliers, replace=False)


def gen_weight(w: Workload) -> np.ndarray:
    """Weight [d_out, d_in] (the nn.Linear convention, K contiguous)."""
    return _cast(rng(w.key, S_W).normal(0.0, w.w_std, (w.d_out, w.d_in)), w.dtype)


def gen_bias(w: Workload) -> np.ndarray:
    """Bias [d_out], always fp32."""
    return rng(w.key, S_B).normal(0.0, w.b_std, w.d_out).astype(np.float32)


def gen_lowrank(w: Workload):
    """(L1 [d_in, r], L2 [r, d_out]) in the workload dtype, or (None, None)."""
    if w.rank == 0:
        return None, None
    l1 = _cast(rng(w.key, S_L1).normal(0.0, w.lr_std, (w.d_in, w.rank)), w.dtype)
    l2 = _cast(rng(w.key, S_L2).normal(0.0, w.lr_std, (w.rank, w.d_out)), w.dtype)
    return l1, l2


def custom(key: int, T: int, d_in: int, d_out: int, *, dtype: str = "f32", block: int = 0,
           alpha: Optional[float] = 0.5, center: int = 1, a_bits: int = 4, w_bits: int = 4,
           rank: int = 0, x_dist: str = "normal", n_outliers: int = 0,
           outlier: float = 50.0, w_std: float = 0.02, group: int = 0) -> Workload:
    """An ad-hoc workload for edge-case and ragged-shape tests."""
    return Workload(key, f"custom{key}", T, d_in, d_out, dtype, block or d_in, alpha, center,
                    a_bits, w_bits, rank, x_dist, n_outliers, outlier, outlier, w_std,
                    group=group)


def generate(w: Workload, T: Optional[int] = None):
    """All inputs of workload ``w`` as a dict of numpy arrays."""
    l1, l2 = gen_lowrank(w)
    return {"x": gen_x(w, T), "weight": gen_weight(w), "bias": gen_bias(w), "l1": l1, "l2": l2}
