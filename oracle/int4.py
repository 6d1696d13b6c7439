"""int4 weight decoding (per-row and group-wise), written from the definition.  TEST INFRASTRUCTURE.

[LOG-g4] describes two int4 containers that share one packing: fmt=2 (per-row,
one scale per output row) and fmt=4 (group-wise, O*ceil(C/gs) scales, gs even so
a packed byte never holds two groups, gs=0 meaning per-row).  Nibbles are
offset-binary ("offset->signed nibble conversion" happens at upload), so a
nibble q stands for the integer q - 8.

Readings (pages silent):
* low nibble of byte b holds the even column 2b, high nibble the odd column 2b+1;
* the last group of a row is C - gs*(ceil(C/gs)-1) columns wide and has its own
  scale (the pages test a 200 % 64 tail);
* gs >= C gives a single group per row.
"""

from __future__ import annotations

import numpy as np

FMT_ROW = 2
FMT_GROUP = 4


def check_format(fmt: int, gs: int, O: int, C: int) -> None:
    """Reject what [LOG-g4] says must not be decoded: unknown fmt codes, odd gs, odd C."""
    if fmt not in (FMT_ROW, FMT_GROUP):
        raise ValueError(f"unsupported fmt {fmt}")
    if O <= 0 or C <= 0 or C % 2:
        raise ValueError(f"bad shape {O}x{C}")
    if fmt == FMT_GROUP and (gs < 0 or gs % 2):
        raise ValueError(f"group size must be even and >= 0, got {gs}")
    if fmt == FMT_ROW and gs != 0:
        raise ValueError("per-row tensors take gs = 0")


def n_groups(fmt: int, gs: int, C: int) -> int:
    """Scales per row: 1 for per-row (fmt=2, or fmt=4 with gs=0), else ceil(C/gs) [LOG-g4]."""
    if fmt == FMT_GROUP and gs > 0:
        return -(-C // gs)
    return 1


def unpack_nibbles(packed: np.ndarray, O: int, C: int) -> np.ndarray:
    """uint8 [O, C//2] -> nibble codes q in 0..15, uint8 [O, C].  Column 2b = low nibble of byte b."""
    p = np.asarray(packed, dtype=np.uint8).reshape(O, C // 2)
    q = np.empty((O, C), dtype=np.uint8)
    q[:, 0::2] = p & 0x0F
    q[:, 1::2] = p >> 4
    return q


def scale_matrix(scales: np.ndarray, fmt: int, gs: int, O: int, C: int, rows=None) -> np.ndarray:
    """f64 [len(rows), C]: the scale that multiplies each weight (column c lies in group c // gs)."""
    rows = np.arange(O) if rows is None else np.asarray(rows)
    ng = n_groups(fmt, gs, C)
    s = np.asarray(scales, dtype=np.float32).astype(np.float64).reshape(O, ng)[rows]
    if ng == 1:
        return np.repeat(s, C, axis=1)
    col_group = np.arange(C) // gs
    return s[:, col_group]


def dequantize_rows(packed, scales, fmt: int, gs: int, O: int, C: int, rows) -> np.ndarray:
    """W[o, c] = (q[o, c] - 8) * scale(o, c) in f64, for the listed rows only."""
    check_format(fmt, gs, O, C)
    rows = np.asarray(rows)
    p = np.asarray(packed, dtype=np.uint8).reshape(O, C // 2)[rows]
    q = unpack_nibbles(p, len(rows), C).astype(np.float64) - 8.0
    return q * scale_matrix(scales, fmt, gs, O, C, rows)


def dequantize(packed, scales, fmt: int, gs: int, O: int, C: int) -> np.ndarray:
    """Whole tensor, f64 [O, C]."""
    return dequantize_rows(packed, scales, fmt, gs, O, C, np.arange(O))


def matvec_rows(t, v: np.ndarray, rows=None, block: int = 1024) -> np.ndarray:
    """(W v)[rows] in f64 for a tensor t with fields fmt, gs, O, C, packed, scales.

    A library matmul is the contraction step; rows are decoded in blocks only to
    bound memory."""
    rows = np.arange(t.O) if rows is None else np.asarray(rows)
    v = np.asarray(v, dtype=np.float64)
    out = np.empty((len(rows),) + v.shape[1:], dtype=np.float64)
    for i in range(0, len(rows), block):
        r = rows[i:i + block]
        out[i:i + block] = dequantize_rows(t.packed, t.scales, t.fmt, t.gs, t.O, t.C, r) @ v
    return out
