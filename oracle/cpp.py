"""ctypes face of the C++17 CPU oracle (oracle/hq_oracle.cpp).

TEST INFRASTRUCTURE ONLY, like oracle/hq_oracle.py: the tests, the entry
point's smoke check and the benchmark's CPU-baseline leg use it, nothing in
the library's product path. It shares no code with the HIP path.

build() compiles the shared library with the host compiler (g++ -O2,
pthreads); load() opens it. The functions take and return NumPy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "hq_oracle.cpp")
LIB = os.path.join(HERE, "libhqoracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile oracle/libhqoracle.so with g++ (every call recompiles)."""
    tmp = LIB + ".tmp"
    cmd = ["g++", "-O2", "-std=c++17", "-shared", "-fPIC", "-pthread", SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"g++ failed on {SRC}:\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB):
        raise RuntimeError(f"{LIB} is not built; run oracle.cpp.build()")
    lib = ctypes.CDLL(LIB)
    P = ctypes.c_void_p
    I, I64 = ctypes.c_int, ctypes.c_int64
    lib.hqo_prepare.restype = I
    lib.hqo_prepare.argtypes = [I, I, I, I, P, P, P, P, P, I]
    lib.hqo_quant_linear.restype = I
    lib.hqo_quant_linear.argtypes = [I64, I, I, I, I, I, P, P, P, P, P, P, I, P, P, I, P, P, P,
                                     P, P, I]
    lib.hqo_rotate.restype = I
    lib.hqo_rotate.argtypes = [I64, I, I, P, P]
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f64(a):
    return None if a is None else np.ascontiguousarray(a, dtype=np.float64)


def default_threads() -> int:
    return len(os.sched_getaffinity(0))


def rotate(x, block: int) -> np.ndarray:
    """Rows of x times the block-diagonal normalised Sylvester matrix."""
    x = _f64(x)
    out = np.empty_like(x)
    st = load().hqo_rotate(x.shape[0], x.shape[1], block, _p(x), _p(out))
    if st:
        raise ValueError(f"hqo_rotate failed ({st})")
    return out


def prepare_weights(weight, sigma, block: int, w_bits: int, threads: int = 0):
    """W~ codes, s_w and c (as the Python oracle's prepare_weights, without W~)."""
    weight = _f64(weight)
    d_out, d_in = weight.shape
    sigma = _f64(sigma)
    qw = np.empty((d_out, d_in), dtype=np.int16)
    s_w = np.empty(d_out)
    c = np.empty(d_out)
    st = load().hqo_prepare(d_in, d_out, block, w_bits, _p(weight), _p(sigma), _p(qw), _p(s_w),
                            _p(c), threads or default_threads())
    if st:
        raise ValueError(f"hqo_prepare failed ({st})")
    return {"qw": qw, "s_w": s_w, "c": c}


def quant_linear(x, prepared, bias, sigma, *, block: int, a_bits: int, center: int,
                 l1=None, l2=None, out_dtype: str = "f32", want_acc: bool = True,
                 threads: int = 0):
    """Online half for the rows of x: codes, scales, means, accumulators and
    Y rounded to out_dtype ("f32" or "bf16")."""
    x = _f64(x)
    T, d_in = x.shape
    qw = np.ascontiguousarray(prepared["qw"], dtype=np.int16)
    d_out = qw.shape[0]
    rank = 0 if l1 is None else np.asarray(l1).shape[1]
    qa = np.empty((T, d_in), dtype=np.int16)
    s_x = np.empty(T)
    mu = np.empty(T)
    acc = np.empty((T, d_out), dtype=np.int64) if want_acc else None
    y = np.empty((T, d_out))
    l1, l2 = _f64(l1), _f64(l2)
    st = load().hqo_quant_linear(
        T, d_in, d_out, block, a_bits, int(center), _p(x), _p(_f64(sigma)), _p(qw),
        _p(_f64(prepared["s_w"])), _p(_f64(prepared["c"])), _p(_f64(bias)), rank, _p(l1),
        _p(l2), 1 if out_dtype == "bf16" else 0, _p(qa), _p(s_x), _p(mu), _p(acc), _p(y),
        threads or default_threads())
    if st:
        raise ValueError(f"hqo_quant_linear failed ({st})")
    return {"qa": qa, "s_x": s_x, "mu": mu, "acc": acc, "y_out": y}
