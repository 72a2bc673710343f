"""Host-side reader and writer of libhq's code formats, written from their
definition in include/hq.h ("Code formats"), for the tests only.

* HQ_CODES_I8: int8 bytes, row-major [rows, d].
* HQ_CODES_E2M3: each code q in [-7, 7] as the 6-bit float E2M3 of the same
  value (sign bit 5, exponent bits 4..3 with bias 1, mantissa bits 2..0);
  rows in groups of 4, group g at byte 3 d g, 128-code slice s of row 4g + i
  at byte 384 s + 96 i inside it, code k of the slice at bits [6k, 6k + 6) of
  that 96-byte little-endian string.

The E2M3 decoder evaluates the float definition and checks that every value
is an integer in [-7, 7]; it shares nothing with the library's encoder.
"""
import numpy as np

I8, E2M3 = 0, 1
RG = 4            # rows per E2M3 row group


def fmt_of(a_bits: int, w_bits: int, gemm: int = 0) -> int:
    return E2M3 if (a_bits == 4 and w_bits == 4 and gemm == 0) else I8


def nbytes(fmt: int, rows: int, d: int) -> int:
    if fmt == E2M3:
        return (rows + RG - 1) // RG * (RG * 3 // 4) * d
    return rows * d


def e2m3_value(bits: np.ndarray) -> np.ndarray:
    """Float value of 6-bit E2M3 patterns (the format's definition)."""
    b = bits.astype(np.int64)
    sign = np.where(b & 0x20, -1.0, 1.0)
    e = (b >> 3) & 0x3
    m = (b & 0x7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0, np.ldexp(1.0 + m / 8.0, (e - 1).astype(np.int64)))
    return sign * mag


def e2m3_bits(q: np.ndarray) -> np.ndarray:
    """E2M3 pattern of integer codes in [-7, 7] (searched in the value table)."""
    table = e2m3_value(np.arange(32))           # non-negative patterns 0..31
    q = np.asarray(q, dtype=np.int64)
    assert np.all(np.abs(q) <= 7)
    mag = np.abs(q)
    pat = np.array([int(np.flatnonzero(table == v)[0]) for v in range(8)], dtype=np.int64)[mag]
    return np.where(q < 0, pat | 0x20, pat)


def decode(fmt: int, buf, rows: int, d: int, idx=None) -> np.ndarray:
    """int64 codes [rows, d] from a code buffer (numpy uint8 or int8) of
    `rows` rows; with `idx`, only those rows (in that order)."""
    raw = np.ascontiguousarray(np.asarray(buf).view(np.uint8).reshape(-1))
    assert raw.size >= nbytes(fmt, rows, d), (raw.size, nbytes(fmt, rows, d))
    idx = np.arange(rows) if idx is None else np.asarray(idx, dtype=np.int64)
    assert idx.size == 0 or (idx.min() >= 0 and idx.max() < rows)
    if fmt == I8:
        return raw[:rows * d].view(np.int8).reshape(rows, d)[idx].astype(np.int64)
    S = d // 128
    base = ((idx // RG)[:, None] * (RG * 3 // 4 * d) + np.arange(S)[None, :] * (96 * RG)
            + (idx % RG)[:, None] * 96)
    seg = raw[base[..., None] + np.arange(96)]                        # [n, S, 96]
    bits = np.unpackbits(seg, axis=-1, bitorder="little").reshape(idx.size, S, 128, 6)
    pat = (bits.astype(np.int64) << np.arange(6)).sum(axis=-1)       # [n, S, 128]
    val = e2m3_value(pat)
    q = np.rint(val).astype(np.int64)
    assert np.all(val == q) and np.all(np.abs(q) <= 7), "non-integer E2M3 code"
    return q.reshape(idx.size, d)


def encode(fmt: int, codes: np.ndarray) -> np.ndarray:
    """Code buffer (numpy uint8) of integer codes [rows, d]."""
    codes = np.asarray(codes)
    rows, d = codes.shape
    if fmt == I8:
        return codes.astype(np.int8).view(np.uint8).reshape(-1).copy()
    groups = (rows + RG - 1) // RG
    gb = RG * 3 // 4 * d                             # bytes per group
    out = np.empty(groups * gb, dtype=np.uint8)
    step = 256                                       # groups per chunk (bounded memory)
    for g0 in range(0, groups, step):
        g1 = min(groups, g0 + step)
        full = np.zeros(((g1 - g0) * RG, d), dtype=np.int64)
        part = codes[g0 * RG:min(rows, g1 * RG)]
        full[:part.shape[0]] = part
        pat = e2m3_bits(full).reshape(g1 - g0, RG, d // 128, 128).transpose(0, 2, 1, 3)
        bits = ((pat[..., None] >> np.arange(6)) & 1).astype(np.uint8)
        seg = np.packbits(bits.reshape(g1 - g0, d // 128, RG, 768), axis=-1, bitorder="little")
        out[g0 * gb:g1 * gb] = seg.reshape(-1)
    return out
