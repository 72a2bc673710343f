"""Host-side tests of the C ABI: the library loads, exports every declared
symbol, and rejects bad arguments before touching the GPU. No kernels run."""
import ctypes

import pytest

from hadamard_rotated_bit_amd import _lib
from hadamard_rotated_bit_amd import Desc, F32, BF16
from hadamard_rotated_bit_amd import workloads as WL
import codefmt

lib = _lib.load()


def _d(**kw):
    base = dict(d_in=1152, d_out=4608, block=128, a_bits=4, w_bits=4, center=True, smooth=True,
                rank=0, x_dtype=BF16, w_dtype=BF16, y_dtype=BF16)
    base.update(kw)
    return Desc(**base).c()


def test_exports_every_declared_function():
    names = _lib.header_functions()
    assert len(names) >= 16
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_status_strings():
    assert lib.hq_abi_version() == 8
    assert lib.hq_status_str(0) == b"HQ_OK"
    assert lib.hq_status_str(-3) == b"HQ_ERR_WORKSPACE"
    assert lib.hq_status_str(99) == b"HQ_ERR_UNKNOWN"


@pytest.mark.parametrize("name", WL.ORDER)
def test_workload_descriptors_valid(name):
    w = WL.WORKLOADS[name]
    dt = BF16 if w.dtype == "bf16" else F32
    d = Desc(w.d_in, w.d_out, w.block, w.a_bits, w.w_bits, bool(w.center), w.alpha is not None,
             w.rank, dt, dt, dt).c()
    assert lib.hq_validate(ctypes.byref(d)) == 0
    L = _lib.HqLayout()
    assert lib.hq_prepared_layout_of(ctypes.byref(d), ctypes.byref(L)) == 0
    assert L.d_out_pad % 256 == 0 and L.d_out_pad >= w.d_out
    offs = [L.w_codes, L.w_scale, L.c, L.bias, L.sigma_inv, L.l1_hi, L.l1_lo, L.l2_hi, L.l2_lo]
    assert all(o % 256 == 0 for o in offs) and offs == sorted(offs)
    fmt = codefmt.fmt_of(w.a_bits, w.w_bits)
    assert lib.hq_code_format(ctypes.byref(d)) == fmt
    assert L.w_scale - L.w_codes >= codefmt.nbytes(fmt, L.d_out_pad, w.d_in)
    assert L.total == lib.hq_prepared_bytes(ctypes.byref(d))
    ws = lib.hq_workspace_bytes(ctypes.byref(d), w.T)
    assert ws >= codefmt.nbytes(fmt, w.T, w.d_in) + 8 * w.T + 4 * w.T * w.rank


@pytest.mark.parametrize("kw,status", [
    (dict(d_in=0), -1), (dict(d_out=-8), -1), (dict(x_dtype=3), -1), (dict(center=3), -1), (dict(center=-1), -1),
    (dict(smooth=5), -1), (dict(a_bits=3), -2), (dict(w_bits=16), -2), (dict(d_in=1000), -2),
    (dict(d_in=2176), -2), (dict(d_out=100), -2), (dict(block=96), -2), (dict(block=256, d_in=1152), -2),
    (dict(rank=8), -2), (dict(rank=128), -2), (dict(d_in=16384), -2), (dict(gemm=2), -1),
    (dict(gemm=-1), -1), (dict(group=32), -2), (dict(group=128), -2), (dict(group=-64), -2),
    (dict(group=64, a_bits=8), -2), (dict(group=64, w_bits=8), -2), (dict(group=64, gemm=1), -2),
])
def test_validation_rejects(kw, status):
    d = _d(**kw)
    assert lib.hq_validate(ctypes.byref(d)) == status
    assert len(lib.hq_last_error()) > 0
    assert lib.hq_prepared_bytes(ctypes.byref(d)) == 0
    assert lib.hq_workspace_bytes(ctypes.byref(d), 16) == 0


@pytest.mark.parametrize("d_in", [128, 256, 384, 1152, 2048, 2560, 3072, 4096, 6144, 8192])
def test_supported_widths(d_in):
    assert lib.hq_validate(ctypes.byref(_d(d_in=d_in, block=128))) == 0


def test_block_one_and_full():
    assert lib.hq_validate(ctypes.byref(_d(block=1))) == 0
    assert lib.hq_validate(ctypes.byref(_d(d_in=4096, block=4096))) == 0


@pytest.mark.parametrize("a_bits,w_bits,gemm,fmt", [(4, 4, 0, 1), (8, 4, 0, 0), (4, 8, 0, 0),
                                                    (8, 8, 0, 0), (4, 4, 1, 0), (8, 8, 1, 0)])
def test_code_format_and_bytes(a_bits, w_bits, gemm, fmt):
    d = ctypes.byref(_d(a_bits=a_bits, w_bits=w_bits, gemm=gemm))
    assert lib.hq_code_format(d) == fmt
    for rows in [0, 1, 3, 4, 5, 8192]:
        assert lib.hq_code_bytes(d, rows) == codefmt.nbytes(fmt, rows, 1152)
    assert lib.hq_code_bytes(d, -1) == 0
    assert lib.hq_code_format(ctypes.byref(_d(a_bits=5))) == -2


def test_e2m3_table_matches_format_definition():
    # codes 0..7 and their negatives against the E2M3 definition (sign, two
    # exponent bits with bias 1, three mantissa bits), and the sample of the
    # format text: |q| = 0..7 -> 0, 8, 16, 20, 24, 26, 28, 30
    import numpy as np
    pats = codefmt.e2m3_bits(np.arange(-7, 8))
    assert list(pats[7:]) == [0, 8, 16, 20, 24, 26, 28, 30]
    assert list(codefmt.e2m3_value(pats)) == list(range(-7, 8))
    assert codefmt.e2m3_value(np.array([0b000100]))[0] == 0.5      # subnormal m/8
    assert codefmt.e2m3_value(np.array([0b011111]))[0] == 7.5      # largest
    # a hand-packed 128-code slice: code 0 = 1, code 1 = -7
    q = np.zeros((1, 128), dtype=np.int64)
    q[0, 0], q[0, 1] = 1, -7
    buf = codefmt.encode(codefmt.E2M3, q)
    assert buf.size == 384 and buf[0] == 0x88 and buf[1] == 0x0F and not buf[2:].any()


def test_e2m3_row_group_placement():
    # the layout text's offsets, element by element: code k of row 4g + i sits
    # in slice s = k // 128 at byte 3 d g + 384 s + 96 i, bits 6 (k % 128) up
    import numpy as np
    d, rows = 256, 70
    q = np.zeros((rows, d), dtype=np.int64)
    for r, k, v in [(0, 0, 3), (37, 130, -5), (69, 255, 7), (31, 127, -1)]:
        q[r, k] = v
    buf = codefmt.encode(codefmt.E2M3, q)
    assert buf.size == 18 * 3 * d
    pat = codefmt.e2m3_bits(np.array([3, -5, 7, -1]))
    for (r, k), p in zip([(0, 0), (37, 130), (69, 255), (31, 127)], pat):
        g, i, s, kk = r // 4, r % 4, k // 128, k % 128
        bit = 8 * (3 * d * g + 384 * s + 96 * i) + 6 * kk
        got = sum(((int(buf[(bit + j) // 8]) >> ((bit + j) % 8)) & 1) << j for j in range(6))
        assert got == p
    np.testing.assert_array_equal(codefmt.decode(codefmt.E2M3, buf, rows, d), q)


@pytest.mark.parametrize("d_in,rank,T,slices", [
    (3072, 32, 300, 8), (3072, 32, 4200, 6), (3072, 32, 4608, 6), (3072, 32, 65536, 6),
    (3072, 16, 4500, 6), (3072, 48, 4608, 0), (2048, 32, 128, 8), (2048, 32, 8192, 4),
    (1152, 16, 8192, 4), (4096, 32, 4608, 8)])
def test_low_rank_slice_count(d_in, rank, T, slices):
    # The workspace holds U [T, rank] and the slice products [slices, T, rank]
    # of the two-pass down projection. The slice count is the one of 4, 6
    # and 8 (whole 32-channel steps, at most 16 steps per slice, the slice of
    # L1 within one block's registers and LDS) with the least channels per
    # slice times rounds of 128-row blocks over 256 compute units, fewer
    # slices on a tie: d_in 3072 takes 8 slices of 384 at 300 rows (one
    # round either way) and 6 slices of 512 from 33 blocks of rows up; rank
    # 48 at 3072 fits no slicing (one-pass form, no slice products).
    with_r = _d(d_in=d_in, block=128, rank=rank)
    without = _d(d_in=d_in, block=128, rank=0)
    assert lib.hq_validate(ctypes.byref(with_r)) == 0
    al = lambda n: (n + 255) // 256 * 256
    extra = lib.hq_workspace_bytes(ctypes.byref(with_r), T) - \
        lib.hq_workspace_bytes(ctypes.byref(without), T)
    assert extra == al(4 * T * rank) + al(4 * slices * T * rank)


@pytest.mark.parametrize("w_dtype,esize", [(BF16, 2), (F32, 4)])
def test_channel_centring_layout(w_dtype, esize):
    # center = 2 keeps a copy of the weight in the blob and needs partial sums,
    # the channel mean and the corrected bias in the workspace
    tok = _d(w_dtype=w_dtype)
    chan = _d(center=2, w_dtype=w_dtype)
    assert lib.hq_validate(ctypes.byref(chan)) == 0
    Lt, Lc = _lib.HqLayout(), _lib.HqLayout()
    assert lib.hq_prepared_layout_of(ctypes.byref(tok), ctypes.byref(Lt)) == 0
    assert lib.hq_prepared_layout_of(ctypes.byref(chan), ctypes.byref(Lc)) == 0
    assert Lt.weight == 0 and Lc.weight % 256 == 0 and Lc.weight >= Lc.l2_lo
    assert Lc.total - Lc.weight >= esize * 4608 * 1152
    for T in [1, 64, 65, 8192]:
        extra = lib.hq_workspace_bytes(ctypes.byref(chan), T) - \
            lib.hq_workspace_bytes(ctypes.byref(tok), T)
        chunks = (T + 63) // 64
        assert extra >= 4 * (chunks * 1152 + 1152 + Lc.d_out_pad)


@pytest.mark.parametrize("center", [0, 1, 2])
def test_group_layout(center):
    # group = 64: one weight scale per output channel and group in the blob
    # ([d_in / 64, d_out_pad], group-major) and one activation scale per token
    # and group in the workspace
    row = _d(center=center, d_in=3072, block=64)
    grp = _d(center=center, d_in=3072, block=64, group=64)
    assert lib.hq_validate(ctypes.byref(grp)) == 0
    assert lib.hq_code_format(ctypes.byref(grp)) == _lib.HQ_CODES_E2M3
    Lr, Lg = _lib.HqLayout(), _lib.HqLayout()
    assert lib.hq_prepared_layout_of(ctypes.byref(row), ctypes.byref(Lr)) == 0
    assert lib.hq_prepared_layout_of(ctypes.byref(grp), ctypes.byref(Lg)) == 0
    G = 3072 // 64
    assert Lg.c - Lg.w_scale >= 4 * G * Lg.d_out_pad
    assert Lg.total - Lr.total == (Lg.c - Lg.w_scale) - (Lr.c - Lr.w_scale)
    for T in [1, 64, 65, 4608]:
        extra = lib.hq_workspace_bytes(ctypes.byref(grp), T) - \
            lib.hq_workspace_bytes(ctypes.byref(row), T)
        a256 = lambda n: (n + 255) // 256 * 256
        assert extra == a256(4 * G * T) - a256(4 * T)


def test_group_desc_python_mirror():
    d = Desc(3072, 12288, 64, group=64)
    assert d.c().group == 64
    assert d.sx_shape(10) == (48, 10)
    assert Desc(3072, 12288, 64).sx_shape(10) == (10,)


def test_channel_center_rejects_other_modes():
    d = _d(center=1)
    z = ctypes.c_void_p(16)
    assert lib.hq_channel_center(ctypes.byref(d), z, z, 4, z, z, z, 1 << 20, None) == -1
    assert b"center = 2" in lib.hq_last_error()
    c = _d(center=2)
    assert lib.hq_channel_center(ctypes.byref(c), z, z, 0, z, z, z, 1 << 20, None) == -1
    assert lib.hq_channel_center(ctypes.byref(c), z, z, 4, z, z, z, 16, None) == -3


def test_null_desc():
    assert lib.hq_validate(None) == -1
    assert lib.hq_prepared_bytes(None) == 0


def test_entry_points_reject_before_launch():
    d = ctypes.byref(_d())
    p = ctypes.c_void_p(0x1000)   # never dereferenced: every call fails validation first
    assert lib.hq_quant_linear(d, None, p, 16, p, p, 1 << 30, None) == -1
    assert lib.hq_quant_linear(d, p, p, -1, p, p, 1 << 30, None) == -1
    assert lib.hq_quant_linear(d, p, p, 16, p, p, 10, None) == -3          # workspace too small
    assert b"workspace" in lib.hq_last_error()
    assert lib.hq_quant_linear(d, p, p, 0, None, None, 0, None) == 0     # T = 0 is a no-op
    assert lib.hq_prepare_weights(d, p, None, None, None, None, p, None) == -1  # smooth needs sigma
    d_ns = ctypes.byref(_d(smooth=False))
    assert lib.hq_prepare_weights(d_ns, p, None, p, None, None, p, None) == -1  # sigma w/o smooth
    d_r = ctypes.byref(_d(rank=32))
    assert lib.hq_prepare_weights(d_r, p, None, p, None, None, p, None) == -1  # rank needs L1/L2
    assert lib.hq_sigma(d, p, p, ctypes.c_float(1.5), p, None) == -1
    assert lib.hq_gemm_i32(d, p, p, 16, 12, p, None) == -1                # N % 8
    assert lib.hq_gemm_i32(d, p, None, 16, 16, p, None) == -1             # NULL codes
    assert lib.hq_act_quantize(d_r, p, p, 4, p, p, p, None, None) == -1    # U missing
    assert lib.hq_channel_absmax(d, None, 8, p, None) == -1


def test_error_string_is_thread_local():
    import threading
    lib.hq_validate(ctypes.byref(_d(a_bits=3)))
    seen = []
    t = threading.Thread(target=lambda: seen.append(lib.hq_last_error()))
    t.start()
    t.join()
    assert seen == [b""]
    assert b"a_bits" in lib.hq_last_error()


# ---- integer-only DH / WH layers (host-side checks only)

def _il(**kw):
    from hadamard_rotated_bit_amd import IntDesc
    base = dict(d_in=256, d_out=256, block=256, w_dtype=F32)
    base.update(kw)
    return IntDesc(**base)


@pytest.mark.parametrize("kw,status", [
    (dict(d_in=0), -1), (dict(d_out=-8), -1), (dict(w_dtype=4), -1), (dict(d_in=100), -2),
    (dict(d_out=260), -2), (dict(block=3), -2), (dict(block=512, d_out=512), -2),
    (dict(block=128, d_out=200), -2), (dict(block=0), -2), (dict(side=2), -1),
    (dict(side=-1), -1), (dict(in_block=2), -2), (dict(side=1, in_block=3), -2),
    (dict(side=1, in_block=16384), -2), (dict(side=1, in_block=0), -2),
    (dict(side=1, in_block=256, block=512, d_out=200), -2),   # DH pads through post_block
    (dict(block=512, d_out=200), -2), (dict(side=1, d_in=100, in_block=64), -2),
    (dict(act=4), -1), (dict(act=-1), -1), (dict(post_block=3), -2), (dict(post_block=0), -2),
    (dict(post_block=512, d_out=512), -2), (dict(post_block=64, d_out=96, block=1), -2),
    (dict(side=1, in_block=256, act=1, block=16), -2),
])
def test_int_validation_rejects(kw, status):
    d = _il(**kw)
    assert lib.hq_int_validate(d._ref) == status
    assert len(lib.hq_last_error()) > 0
    assert lib.hq_int_prepared_bytes(d._ref) == 0
    assert lib.hq_int_workspace_bytes(d._ref, 16) == 0


@pytest.mark.parametrize("kw", [dict(), dict(side=1, in_block=256), dict(side=1, in_block=1, block=1),
                                dict(side=1, in_block=32, block=8, d_out=136),
                                dict(act=1, post_block=256), dict(act=3, post_block=8, block=16),
                                dict(side=1, in_block=256, act=2, block=1, post_block=64),
                                dict(side=1, in_block=512), dict(side=1, d_in=200, in_block=256),
                                dict(block=256, d_out=200), dict(post_block=256, d_out=200),
                                dict(block=256, d_out=200, act=3, post_block=256)])
def test_int_validation_accepts(kw):
    assert lib.hq_int_validate(_il(**kw)._ref) == 0


def test_int_padded_layout_and_workspace():
    # a WH layer with a padded output order (200 channels, H_256) holds 256
    # accumulator rows; a DH layer with a padded input order (200 -> 256)
    # takes 256 input codes per token
    d = _il(d_in=384, d_out=200, block=256)
    L = _lib.HqIntLayout()
    assert lib.hq_int_prepared_layout_of(d._ref, ctypes.byref(L)) == 0
    assert L.d_out_pad == 256 and L.w_scale - L.w_codes >= 256 * 384
    assert L.total - L.wbar >= 4 * 256 * 384
    assert lib.hq_int_workspace_bytes(d._ref, 10) == 4 * 10 * 256 + (256 - (4 * 10 * 256) % 256) % 256
    p = _il(d_in=200, d_out=64, block=1, side=1, in_block=256)
    assert lib.hq_int_prepared_layout_of(p._ref, ctypes.byref(L)) == 0
    assert L.w_scale - L.w_codes >= 256 * L.d_out_pad
    assert (p.x_width, p.acc_width, p.out_width) == (256, 64, 64)
    q = _il(d_out=200, block=256, post_block=256, act=1)
    assert (q.x_width, q.acc_width, q.out_width) == (256, 256, 256)


def test_int_layout_and_workspace():
    d = _il(d_in=384, d_out=136, block=8)
    assert lib.hq_int_validate(d._ref) == 0
    L = _lib.HqIntLayout()
    assert lib.hq_int_prepared_layout_of(d._ref, ctypes.byref(L)) == 0
    assert L.d_out_pad == 256
    offs = [L.w_codes, L.w_scale, L.b_int, L.mult, L.shift, L.lut, L.wbar, L.total]
    assert all(o % 256 == 0 for o in offs[:-1]) and offs == sorted(offs)
    assert (L.mult_in, L.shift_in) == (L.shift + 4, L.shift + 8) and L.wbar - L.lut >= 256
    assert L.w_scale - L.w_codes >= 256 * 384 and L.total - L.wbar >= 4 * 136 * 384
    assert L.b_int - L.w_scale >= 4 * 256 and L.mult - L.b_int >= 4 * 256
    assert lib.hq_int_prepared_bytes(d._ref) == L.total
    assert lib.hq_int_workspace_bytes(d._ref, 1000) == 4 * 1000 * 136
    assert lib.hq_int_workspace_bytes(d._ref, -1) == 0


def test_int_entry_points_reject_before_launch():
    d = _il()._ref
    p = ctypes.c_void_p(0x1000)   # never dereferenced: every call fails validation first
    f = ctypes.c_float
    assert lib.hq_int_prepare(d, None, None, f(1.0), f(1.0), f(0.0), f(0.0), p, None) == -1
    assert lib.hq_int_prepare(d, p, None, f(0.0), f(1.0), f(0.0), f(0.0), p, None) == -1
    assert lib.hq_int_prepare(d, p, None, f(1.0), f(float("nan")), f(0.0), f(0.0), p,
                              None) == -1
    # a SiLU / GELU table needs both of its grids
    g = _il(act=3, post_block=8)._ref
    assert lib.hq_int_prepare(g, p, None, f(1.0), f(1.0), f(0.0), f(1.0), p, None) == -1
    assert lib.hq_int_prepare(g, p, None, f(1.0), f(1.0), f(1.0), f(float("inf")), p,
                              None) == -1
    assert lib.hq_int_linear(d, p, p, -1, p, p, 1 << 30, None) == -1
    assert lib.hq_int_linear(d, p, p, 16, p, p, 10, None) == -3
    assert lib.hq_int_linear(d, p, p, 0, None, None, 0, None) == 0
    assert lib.hq_int_linear(d, None, p, 16, p, p, 1 << 30, None) == -1
    assert lib.hq_int_requant(d, p, None, 16, p, None) == -1
    assert lib.hq_int_requant(d, p, ctypes.c_void_p(0x1001), 16, p, None) == -1   # misaligned


def test_entry_points_reject_misaligned_pointers():
    # every entry point that launches kernels rejects a pointer that is not
    # 16-byte aligned on the host, before anything is enqueued (each call
    # below has exactly one misaligned pointer, so none reaches a launch)
    d = ctypes.byref(_d())
    d_ns = ctypes.byref(_d(smooth=False))
    p = ctypes.c_void_p(0x1000)
    q = ctypes.c_void_p(0x1008)
    f = ctypes.c_float

    def bad(st):
        assert st == -1
        assert b"aligned" in lib.hq_last_error()

    bad(lib.hq_channel_absmax(d, q, 8, p, None))
    bad(lib.hq_channel_absmax(d, p, 8, q, None))
    bad(lib.hq_sigma(d, p, q, f(0.5), p, None))
    bad(lib.hq_prepare_weights(d, q, None, p, None, None, p, None))
    bad(lib.hq_prepare_weights(d, p, None, p, None, None, q, None))
    bad(lib.hq_prepare_weights(d_ns, p, q, None, None, None, p, None))
    bad(lib.hq_quant_linear(d, p, q, 16, p, p, 1 << 30, None))
    bad(lib.hq_quant_linear(d, p, p, 16, q, p, 1 << 30, None))
    bad(lib.hq_act_quantize(d, p, q, 4, p, p, p, None, None))
    bad(lib.hq_act_quantize(d, p, p, 4, q, p, p, None, None))
    bad(lib.hq_act_quantize(d, q, p, 4, p, p, p, None, None))
    bad(lib.hq_act_quantize_ws(d, p, p, 4, p, p, p, None, q, 1 << 30, None))
    bad(lib.hq_act_quantize_ws(d, p, q, 4, p, p, p, None, p, 1 << 30, None))
    bad(lib.hq_act_transform(d, p, q, 4, p, p, None))
    bad(lib.hq_act_transform(d, p, p, 4, q, p, None))
    bad(lib.hq_gemm_i32(d, q, p, 16, 16, p, None))
    bad(lib.hq_gemm_i32(d, p, q, 16, 16, p, None))
    bad(lib.hq_gemm_i32(d, p, p, 16, 16, q, None))
    bad(lib.hq_gemm_dequant(d, p, q, p, p, None, 16, p, None))
    bad(lib.hq_gemm_dequant(d, p, p, p, p, None, 16, q, None))
    c = ctypes.byref(_d(center=2))
    bad(lib.hq_channel_center(c, p, q, 4, p, p, p, 1 << 30, None))
    wi = _il()._ref
    bad(lib.hq_int_prepare(wi, q, None, f(1.0), f(1.0), f(0.0), f(0.0), p, None))
    bad(lib.hq_int_linear(wi, p, q, 16, p, p, 1 << 30, None))


def test_every_declaration_cites_its_passage():
    # each function declared in include/hq.h is preceded by a comment that
    # cites the passage defining its operation (an equation, section, figure
    # or step of the pages), or says that it is bookkeeping of the interface
    # with no step of the method, or names the callers it exists for
    import re
    with open(_lib.HEADER) as f:
        text = f.read()
    cite = re.compile(r"Eq\. \(\d+\)|Sec\. [IVX]+|Fig\. \d|steps? \d|Bookkeeping|cannot allocate")
    decl = re.compile(r"^(?:const\s+)?(?:int|size_t|char|void)\s*\*?\s*(hq_[a-z0-9_]+)\s*\(", re.M)
    seen = 0
    for m in decl.finditer(text):
        head = text[:m.start()]
        comment = head[head.rfind("/*"):]
        assert "*/" in comment, m.group(1)
        # only declarations (and blank lines) may stand between the comment and this one
        between = comment[comment.rfind("*/") + 2:]
        assert all(re.match(r"^\s*$|^(?:const\s+)?(?:int|size_t|char|void)\b.*|^\s+\S.*[,;]$", ln)
                   for ln in between.splitlines()), (m.group(1), between)
        assert cite.search(comment), f"{m.group(1)}: no citation in {comment!r}"
        seen += 1
    assert seen == len(_lib.header_functions())


def test_noalloc_rejects_before_launch():
    # host-side checks of hq_quant_linear_noalloc: invalid descriptor, T < 0,
    # and a workspace beyond the static array, all refused before any launch
    d = ctypes.byref(_d())
    p = ctypes.c_void_p(0x1000)
    assert lib.hq_quant_linear_noalloc(ctypes.byref(_d(a_bits=3)), p, p, 16, p, None) == -2
    assert lib.hq_quant_linear_noalloc(d, p, p, -1, p, None) == -1
    assert lib.hq_quant_linear_noalloc(d, p, p, 0, None, None) == 0
    big = ctypes.byref(_d(d_in=4096, block=4096))
    T = 12000   # 12000 x 3072 bytes of codes alone exceed the 32 MiB array
    assert lib.hq_workspace_bytes(big, T) > (32 << 20)
    assert lib.hq_quant_linear_noalloc(big, p, p, T, p, None) == -3
    assert b"static scratch" in lib.hq_last_error()
