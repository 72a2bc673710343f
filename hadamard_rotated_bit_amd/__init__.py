"""hadamard_rotated_bit_amd: the rotated-and-centred low-bit linear layer on MI355X.

A thin Python face over libhq (include/hq.h). Every step of the layer runs in
the library's HIP kernels; this module only checks tensors, allocates outputs
and workspaces with torch, and passes device pointers and the current stream.

    desc = Desc(d_in=1152, d_out=4608, block=128, a_bits=4, w_bits=4,
                center=True, smooth=True, x_dtype=BF16, w_dtype=BF16, y_dtype=BF16)
    amax = channel_absmax(desc, X_calib)
    sig = sigma(desc, amax, weight, alpha=0.5)
    prep = prepare(desc, weight, bias, sig)
    Y = quant_linear(desc, prep, X)
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional

import torch

from . import _lib
from ._lib import (HQ_CENTER_CHANNEL, HQ_CENTER_NONE, HQ_CENTER_TOKEN, HQ_CODES_E2M3,
                   HQ_CODES_I8, HQ_GEMM_AUTO, HQ_GEMM_I8, HQ_INT_ACT_GELU, HQ_INT_ACT_NONE,
                   HQ_INT_ACT_RELU, HQ_INT_ACT_SILU, HQ_INT_DH, HQ_INT_WH, HqDesc, HqError,
                   HqLayout, check, load)

F32, BF16 = 0, 1
_TORCH = {F32: torch.float32, BF16: torch.bfloat16}
_NAME = {F32: "f32", BF16: "bf16"}


@dataclasses.dataclass(frozen=True)
class Desc:
    """Layer descriptor; mirrors hq_desc. ``center``: 0 / False none, 1 / True
    per-token mean, 2 per-channel mean over the call's tokens (HQ_CENTER_*).
    ``group``: 0 one scale per row, 64 one per row and 64-channel group."""
    d_in: int
    d_out: int
    block: int
    a_bits: int = 4
    w_bits: int = 4
    center: int = HQ_CENTER_TOKEN
    smooth: bool = False
    rank: int = 0
    x_dtype: int = F32
    w_dtype: int = F32
    y_dtype: int = F32
    gemm: int = HQ_GEMM_AUTO
    group: int = 0

    def __post_init__(self):
        raw = HqDesc(self.d_in, self.d_out, self.block, self.a_bits, self.w_bits,
                     int(self.center), int(self.smooth), self.rank, self.x_dtype,
                     self.w_dtype, self.y_dtype, self.gemm, self.group)
        object.__setattr__(self, "_raw", raw)
        object.__setattr__(self, "_ref", ctypes.byref(raw))

    def c(self) -> HqDesc:
        return self._raw

    def sx_shape(self, T: int) -> tuple:
        """Shape of the activation scales of T tokens: (T,), or (d_in / 64, T)
        with group-wise scales (group-major)."""
        return (self.d_in // self.group, T) if self.group else (T,)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def validate(desc: Desc) -> None:
    check(load().hq_validate(desc._ref))


def prepared_bytes(desc: Desc) -> int:
    n = load().hq_prepared_bytes(desc._ref)
    if n == 0:
        check(load().hq_validate(desc._ref))
    return n


def layout(desc: Desc) -> HqLayout:
    out = HqLayout()
    check(load().hq_prepared_layout_of(desc._ref, ctypes.byref(out)))
    return out


def workspace_bytes(desc: Desc, T: int) -> int:
    n = load().hq_workspace_bytes(desc._ref, T)
    if n == 0:
        check(load().hq_validate(desc._ref))
        if T < 0:
            raise HqError(_lib.HQ_ERR_INVALID_ARG, "T must be >= 0")
    return n


def code_format(desc: Desc) -> int:
    """HQ_CODES_I8 or HQ_CODES_E2M3 (see the code formats in include/hq.h)."""
    f = load().hq_code_format(desc._ref)
    if f < 0:
        check(f)
    return f


def code_bytes(desc: Desc, rows: int) -> int:
    """Bytes of a code matrix of `rows` rows in the descriptor's code format."""
    if rows < 0:
        raise HqError(_lib.HQ_ERR_INVALID_ARG, "rows must be >= 0")
    n = load().hq_code_bytes(desc._ref, rows)
    if n == 0 and rows > 0:
        check(load().hq_validate(desc._ref))
    return n


def _need_codes(t: torch.Tensor, name: str, desc: Desc, rows: int) -> None:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype not in (torch.uint8, torch.int8) or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous uint8/int8 code buffer")
    need = code_bytes(desc, rows)
    if t.numel() < need:
        raise ValueError(f"{name} holds {t.numel()} bytes, {need} needed for {rows} rows")


def channel_absmax(desc: Desc, X: torch.Tensor) -> torch.Tensor:
    """Per-input-channel max |X| over tokens (calibration statistic of HadaNorm Eq. (3))."""
    T = X.shape[0]
    _need(X, "X", _TORCH[desc.x_dtype], (T, desc.d_in))
    out = torch.empty(desc.d_in, dtype=torch.float32, device=X.device)
    check(load().hq_channel_absmax(desc._ref, _ptr(X), T, _ptr(out), _stream()))
    return out


def sigma(desc: Desc, act_absmax: torch.Tensor, weight: torch.Tensor, alpha: float) -> torch.Tensor:
    """Smoothing scales sigma_i = max|X_i|^alpha / max|W_i|^(1-alpha) (HadaNorm Eq. (3))."""
    _need(act_absmax, "act_absmax", torch.float32, (desc.d_in,))
    _need(weight, "weight", _TORCH[desc.w_dtype], (desc.d_out, desc.d_in))
    out = torch.empty(desc.d_in, dtype=torch.float32, device=weight.device)
    check(load().hq_sigma(desc._ref, _ptr(act_absmax), _ptr(weight),
                          ctypes.c_float(alpha), _ptr(out), _stream()))
    return out


def prepare(desc: Desc, weight: torch.Tensor, bias: Optional[torch.Tensor] = None,
            sigma: Optional[torch.Tensor] = None, L1: Optional[torch.Tensor] = None,
            L2: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Offline weight transform; returns the prepared blob (uint8 device tensor)."""
    wdt = _TORCH[desc.w_dtype]
    _need(weight, "weight", wdt, (desc.d_out, desc.d_in))
    if bias is not None:
        _need(bias, "bias", torch.float32, (desc.d_out,))
    if sigma is not None:
        _need(sigma, "sigma", torch.float32, (desc.d_in,))
    if L1 is not None:
        _need(L1, "L1", wdt, (desc.d_in, desc.rank))
    if L2 is not None:
        _need(L2, "L2", wdt, (desc.rank, desc.d_out))
    blob = torch.empty(prepared_bytes(desc), dtype=torch.uint8, device=weight.device)
    check(load().hq_prepare_weights(desc._ref, _ptr(weight), _ptr(bias),
                                    _ptr(sigma), _ptr(L1), _ptr(L2), _ptr(blob), _stream()))
    return blob


def check_prepared(desc: Desc, prepared: torch.Tensor) -> None:
    check(load().hq_check_prepared(desc._ref, _ptr(prepared), _stream()))


def quant_linear(desc: Desc, prepared: torch.Tensor, X: torch.Tensor,
                 out: Optional[torch.Tensor] = None,
                 workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Y = the quantised layer applied to X [T, d_in]."""
    T = X.shape[0]
    _need(X, "X", _TORCH[desc.x_dtype], (T, desc.d_in))
    if out is None:
        out = torch.empty(T, desc.d_out, dtype=_TORCH[desc.y_dtype], device=X.device)
    else:
        _need(out, "out", _TORCH[desc.y_dtype], (T, desc.d_out))
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(desc, T), 1), dtype=torch.uint8,
                                device=X.device)
    # the library checks the workspace size itself
    check(load().hq_quant_linear(desc._ref, _ptr(prepared), _ptr(X), T, _ptr(out),
                                 _ptr(workspace), workspace.numel(), _stream()))
    return out


NOALLOC_SCRATCH_BYTES = 32 << 20   # HQ_NOALLOC_SCRATCH_BYTES of include/hq.h


def quant_linear_noalloc(desc: Desc, prepared: torch.Tensor, X: torch.Tensor,
                         out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """quant_linear with the library's static per-GPU scratch array as the
    workspace (hq_quant_linear_noalloc): the call allocates nothing on the
    device besides ``out`` when it is not given. Calls that overlap on one
    GPU share that array and must not run concurrently."""
    T = X.shape[0]
    _need(X, "X", _TORCH[desc.x_dtype], (T, desc.d_in))
    if out is None:
        out = torch.empty(T, desc.d_out, dtype=_TORCH[desc.y_dtype], device=X.device)
    else:
        _need(out, "out", _TORCH[desc.y_dtype], (T, desc.d_out))
    check(load().hq_quant_linear_noalloc(desc._ref, _ptr(prepared), _ptr(X), T, _ptr(out),
                                         _stream()))
    return out


def _channel(desc: Desc) -> bool:
    return int(desc.center) == HQ_CENTER_CHANNEL


def channel_center(desc: Desc, prepared: torch.Tensor, X: torch.Tensor,
                   workspace: Optional[torch.Tensor] = None):
    """Per-channel centring statistics of X (center = 2): (mean [d_in] =
    mean_t(X), bias_eff [d_out_pad] = b + mean_t(X) W)."""
    T = X.shape[0]
    _need(X, "X", _TORCH[desc.x_dtype], (T, desc.d_in))
    mean = torch.empty(desc.d_in, dtype=torch.float32, device=X.device)
    bias_eff = torch.empty(layout(desc).d_out_pad, dtype=torch.float32, device=X.device)
    if workspace is None:
        workspace = torch.empty(max(workspace_bytes(desc, T), 1), dtype=torch.uint8,
                                device=X.device)
    check(load().hq_channel_center(desc._ref, _ptr(prepared), _ptr(X), T, _ptr(mean),
                                   _ptr(bias_eff), _ptr(workspace), workspace.numel(),
                                   _stream()))
    return mean, bias_eff


def channel_center_into(desc: Desc, prepared: torch.Tensor, X: torch.Tensor,
                        mean: torch.Tensor, bias_eff: torch.Tensor,
                        workspace: torch.Tensor) -> None:
    """channel_center writing into preallocated ``mean`` [d_in] and
    ``bias_eff`` [d_out_pad] (no allocation; e.g. under graph capture)."""
    T = X.shape[0]
    _need(X, "X", _TORCH[desc.x_dtype], (T, desc.d_in))
    _need(mean, "mean", torch.float32, (desc.d_in,))
    _need(bias_eff, "bias_eff", torch.float32, (layout(desc).d_out_pad,))
    check(load().hq_channel_center(desc._ref, _ptr(prepared), _ptr(X), T, _ptr(mean),
                                   _ptr(bias_eff), _ptr(workspace), workspace.numel(),
                                   _stream()))


def act_quantize(desc: Desc, prepared: torch.Tensor, X: torch.Tensor, out=None, mean=None,
                 workspace: Optional[torch.Tensor] = None):
    """Activation stage alone: (codes, s_x, mu [T], U [T, rank] or None); s_x
    has desc.sx_shape(T) ([T], or [d_in / 64, T] with group-wise scales).

    ``codes`` is a uint8 buffer of code_bytes(desc, T) bytes in the
    descriptor's code format. ``out`` may supply that tuple preallocated.
    For center = 2 the third entry is the per-channel mean [d_in] that was
    subtracted (``mean`` if given, else channel_center's). With ``workspace``
    (workspace_bytes(desc, T) bytes) the stage runs exactly as inside
    quant_linear (hq_act_quantize_ws: the two-pass low-rank projection);
    without it, hq_act_quantize (one pass, the same bits)."""
    T = X.shape[0]
    _need(X, "X", _TORCH[desc.x_dtype], (T, desc.d_in))
    dev = X.device
    chan = _channel(desc)
    if chan and mean is None:
        mean = channel_center(desc, prepared, X)[0]
    if out is None:
        codes = torch.empty(max(code_bytes(desc, T), 1), dtype=torch.uint8, device=dev)
        s_x = torch.empty(desc.sx_shape(T), dtype=torch.float32, device=dev)
        mu = mean if chan else torch.empty(T, dtype=torch.float32, device=dev)
        U = torch.empty(T, desc.rank, dtype=torch.float32, device=dev) if desc.rank else None
    else:
        codes, s_x, mu, U = out
        if chan:
            mu = mean
        _need_codes(codes, "codes", desc, T)
        _need(s_x, "s_x", torch.float32, desc.sx_shape(T))
        if desc.rank:
            _need(U, "U", torch.float32, (T, desc.rank))
    _need(mu, "mu", torch.float32, (desc.d_in,) if chan else (T,))
    if workspace is None:
        check(load().hq_act_quantize(desc._ref, _ptr(prepared), _ptr(X), T, _ptr(codes),
                                     _ptr(s_x), _ptr(mu), _ptr(U), _stream()))
    else:
        check(load().hq_act_quantize_ws(desc._ref, _ptr(prepared), _ptr(X), T, _ptr(codes),
                                        _ptr(s_x), _ptr(mu), _ptr(U), _ptr(workspace),
                                        workspace.numel(), _stream()))
    return codes, s_x, mu, U


def act_transform(desc: Desc, prepared: torch.Tensor, X: torch.Tensor, mean=None):
    """Float X~ (normalised H, centred) and mu, before quantisation (debug export).
    For center = 2 the second entry is the per-channel mean that was subtracted."""
    T = X.shape[0]
    _need(X, "X", _TORCH[desc.x_dtype], (T, desc.d_in))
    xt = torch.empty(T, desc.d_in, dtype=torch.float32, device=X.device)
    if _channel(desc):
        mu = mean if mean is not None else channel_center(desc, prepared, X)[0]
        _need(mu, "mean", torch.float32, (desc.d_in,))
    else:
        mu = torch.empty(T, dtype=torch.float32, device=X.device)
    check(load().hq_act_transform(desc._ref, _ptr(prepared), _ptr(X), T, _ptr(xt),
                                  _ptr(mu), _stream()))
    return xt, mu


def gemm_i32(desc: Desc, a_codes: torch.Tensor, w_codes: torch.Tensor, T: int,
             N: int) -> torch.Tensor:
    """int32 accumulators [T, N] of a_codes (T rows) . w_codes (N rows)^T, both
    code buffers in the descriptor's code format."""
    _need_codes(a_codes, "a_codes", desc, T)
    _need_codes(w_codes, "w_codes", desc, N)
    acc = torch.empty(T, N, dtype=torch.int32, device=a_codes.device)
    check(load().hq_gemm_i32(desc._ref, _ptr(a_codes), _ptr(w_codes), T, N, _ptr(acc),
                             _stream()))
    return acc


def gemm_dequant(desc: Desc, prepared: torch.Tensor, codes: torch.Tensor, s_x: torch.Tensor,
                 mu: torch.Tensor, U: Optional[torch.Tensor] = None,
                 out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """GEMM + dequant epilogue alone, from act_quantize's outputs (T = the last
    dimension of s_x). For center = 2, ``mu`` is channel_center's bias_eff [d_out_pad]."""
    T = s_x.shape[-1]
    _need_codes(codes, "codes", desc, T)
    _need(s_x, "s_x", torch.float32, desc.sx_shape(T))
    _need(mu, "mu", torch.float32, (layout(desc).d_out_pad,) if _channel(desc) else (T,))
    if desc.rank:
        _need(U, "U", torch.float32, (T, desc.rank))
    Y = out if out is not None else torch.empty(T, desc.d_out, dtype=_TORCH[desc.y_dtype],
                                                device=codes.device)
    _need(Y, "out", _TORCH[desc.y_dtype], (T, desc.d_out))
    check(load().hq_gemm_dequant(desc._ref, _ptr(prepared), _ptr(codes), _ptr(s_x),
                                 _ptr(mu), _ptr(U), T, _ptr(Y), _stream()))
    return Y


def prepared_views(desc: Desc, prepared: torch.Tensor) -> dict:
    """Views of the arrays inside a prepared blob (for inspection and tests);
    w_codes is the raw code buffer of the d_out weight rows."""
    L = layout(desc)
    npad, d = L.d_out_pad, desc.d_in

    def view(off, n, dtype, shape):
        nbytes = n * torch.empty(0, dtype=dtype).element_size()
        return prepared[off:off + nbytes].view(dtype).view(*shape)

    out = {
        "w_codes": prepared[L.w_codes:L.w_codes + code_bytes(desc, desc.d_out)],
        "s_w": (view(L.w_scale, npad * (d // desc.group), torch.float32,
                     (d // desc.group, npad))[:, :desc.d_out] if desc.group
                else view(L.w_scale, npad, torch.float32, (npad,))[:desc.d_out]),
        "c": view(L.c, npad, torch.float32, (npad,))[:desc.d_out],
        "bias": view(L.bias, npad, torch.float32, (npad,))[:desc.d_out],
        "sigma_inv": view(L.sigma_inv, d, torch.float32, (d,)),
    }
    if _channel(desc):
        out["weight"] = view(L.weight, desc.d_out * d, _TORCH[desc.w_dtype], (desc.d_out, d))
    return out


# ---- integer-only DH / WH layers with integer requantisation ---------------

@dataclasses.dataclass(frozen=True)
class IntDesc:
    """Descriptor of an integer-only layer; mirrors hq_int_desc. ``side``
    HQ_INT_WH (weight transformed along its outputs by H of order ``block``)
    or HQ_INT_DH (along its inputs by H of order ``in_block``); ``block`` is
    the order of the output-side integer transform (before the activation),
    ``act`` the activation to the next layer (HQ_INT_ACT_*), ``post_block``
    the order of the transform after it (the next layer's H_in)."""
    d_in: int
    d_out: int
    block: int
    w_dtype: int = F32
    side: int = _lib.HQ_INT_WH
    in_block: int = 1
    act: int = _lib.HQ_INT_ACT_NONE
    post_block: int = 1

    @property
    def x_width(self) -> int:
        """Input codes per token (a padded DH input order takes in_block)."""
        pad = self.side == _lib.HQ_INT_DH and self.in_block > self.d_in
        return self.in_block if pad else self.d_in

    @property
    def acc_width(self) -> int:
        """Accumulator channels (a padded WH output order has block of them)."""
        pad = self.side == _lib.HQ_INT_WH and self.block > self.d_out
        return self.block if pad else self.d_out

    @property
    def out_width(self) -> int:
        """Output codes per token (a padded post order writes post_block)."""
        return self.post_block if self.post_block > self.d_out else self.d_out

    def __post_init__(self):
        raw = _lib.HqIntDesc(self.d_in, self.d_out, self.block, self.w_dtype, self.side,
                             self.in_block, self.act, self.post_block)
        object.__setattr__(self, "_raw", raw)
        object.__setattr__(self, "_ref", ctypes.byref(raw))


def int_layout(desc: IntDesc) -> "_lib.HqIntLayout":
    out = _lib.HqIntLayout()
    check(load().hq_int_prepared_layout_of(desc._ref, ctypes.byref(out)))
    return out


def int_workspace_bytes(desc: IntDesc, T: int) -> int:
    if T < 0:
        raise HqError(_lib.HQ_ERR_INVALID_ARG, "T must be >= 0")
    n = load().hq_int_workspace_bytes(desc._ref, T)
    if n == 0:
        check(load().hq_int_validate(desc._ref))
    return n


def int_prepare(desc: IntDesc, weight: torch.Tensor, bias: Optional[torch.Tensor], s_x: float,
                s_y: float, s_z: float = 0.0, s_u: float = 0.0) -> torch.Tensor:
    """Offline transform of an integer-only layer; returns the prepared blob.
    s_z, s_u: the int8 grids around a SiLU/GELU table (ignored otherwise)."""
    _need(weight, "weight", _TORCH[desc.w_dtype], (desc.d_out, desc.d_in))
    if bias is not None:
        _need(bias, "bias", torch.float32, (desc.d_out,))
    n = load().hq_int_prepared_bytes(desc._ref)
    if n == 0:
        check(load().hq_int_validate(desc._ref))
    blob = torch.empty(n, dtype=torch.uint8, device=weight.device)
    check(load().hq_int_prepare(desc._ref, _ptr(weight), _ptr(bias), ctypes.c_float(s_x),
                                ctypes.c_float(s_y), ctypes.c_float(s_z), ctypes.c_float(s_u),
                                _ptr(blob), _stream()))
    return blob


def int_linear(desc: IntDesc, prepared: torch.Tensor, x_codes: torch.Tensor,
               out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """int8 output codes [T, out_width] of the layer for int8 input codes
    [T, x_width]."""
    T = x_codes.shape[0]
    _need(x_codes, "x_codes", torch.int8, (T, desc.x_width))
    y = out if out is not None else torch.empty(T, desc.out_width, dtype=torch.int8,
                                                device=x_codes.device)
    _need(y, "out", torch.int8, (T, desc.out_width))
    nws = int_workspace_bytes(desc, T)
    ws = workspace if workspace is not None else torch.empty(
        max(nws, 1), dtype=torch.uint8, device=x_codes.device)
    check(load().hq_int_linear(desc._ref, _ptr(prepared), _ptr(x_codes), T, _ptr(y), _ptr(ws),
                               ws.numel(), _stream()))
    return y


def int_requant(desc: IntDesc, prepared: torch.Tensor, acc: torch.Tensor) -> torch.Tensor:
    """Requantisation alone: int8 [T, out_width] from int32 products
    [T, acc_width] (no bias)."""
    T = acc.shape[0]
    _need(acc, "acc", torch.int32, (T, desc.acc_width))
    y = torch.empty(T, desc.out_width, dtype=torch.int8, device=acc.device)
    check(load().hq_int_requant(desc._ref, _ptr(prepared), _ptr(acc), T, _ptr(y), _stream()))
    return y


def int_views(desc: IntDesc, prepared: torch.Tensor) -> dict:
    """Views of the arrays inside an integer-layer prepared blob (for tests)."""
    L = int_layout(desc)
    npad, d, a = L.d_out_pad, desc.x_width, desc.acc_width

    def view(off, n, dtype, shape):
        nbytes = n * torch.empty(0, dtype=dtype).element_size()
        return prepared[off:off + nbytes].view(dtype).view(*shape)

    return {
        "w_codes": view(L.w_codes, npad * d, torch.int8, (npad, d))[:a],
        "s_w": view(L.w_scale, npad, torch.float32, (npad,))[:a],
        "b_int": view(L.b_int, npad, torch.int32, (npad,))[:a],
        "mult": view(L.mult, npad, torch.int32, (npad,))[:a],
        "shift": view(L.shift, 1, torch.int32, (1,)),
        "wbar": view(L.wbar, a * d, torch.float32, (a, d)),
        "lut": view(L.lut, 256, torch.int8, (256,)),
        "mult_in": view(L.mult_in, 1, torch.int32, (1,)),
        "shift_in": view(L.shift_in, 1, torch.int32, (1,)),
    }
