"""Independent exact-arithmetic helpers for pinning the oracle.

Nothing here is taken from the oracle: fp8 values come from torch's float8_e4m3fn
conversion (an independent library routine), bf16 rounding is a nearest-neighbour
search over the sorted list of every bf16 value with exact rational comparison, and
sums are exact Python Fractions.
"""
from __future__ import annotations

import bisect
from fractions import Fraction

import numpy as np
import torch


def fp8_values_torch() -> np.ndarray:
    """fp64 value of every e4m3fn code via torch (NaN for the NaN codes)."""
    codes = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn)
    return codes.to(torch.float64).numpy()


_FP8 = None


def fp8_fraction(code: int) -> Fraction:
    global _FP8
    if _FP8 is None:
        _FP8 = [None if np.isnan(v) else Fraction(float(v)) for v in fp8_values_torch()]
    v = _FP8[code]
    assert v is not None, "NaN code"
    return v


_BF16 = None


def _bf16_table():
    """(sorted exact values of all finite non-negative bf16 patterns, their patterns)."""
    global _BF16
    if _BF16 is None:
        pats = np.arange(0, 0x7F80, dtype=np.uint32)  # +0 .. max finite
        vals = (pats << 16).view(np.float32).astype(np.float64)
        _BF16 = ([Fraction(float(v)) for v in vals], pats.astype(np.uint16))
    return _BF16


def bf16_round_exact(x: Fraction) -> int:
    """bf16 pattern nearest to the exact rational x, ties to the even pattern."""
    vals, pats = _bf16_table()
    sign = 0x8000 if x < 0 else 0
    a = -x if x < 0 else x
    i = bisect.bisect_left(vals, a)
    if i < len(vals) and vals[i] == a:
        return sign | int(pats[i])
    if i >= len(vals):  # above max finite: overflow unless nearer to max
        top = vals[-1]
        ulp = vals[-1] - vals[-2]
        if a - top < ulp / 2:
            return sign | int(pats[-1])
        return sign | 0x7F80
    lo, hi = vals[i - 1], vals[i]
    dlo, dhi = a - lo, hi - a
    if dlo < dhi:
        j = i - 1
    elif dhi < dlo:
        j = i
    else:
        j = i - 1 if int(pats[i - 1]) % 2 == 0 else i
    return sign | int(pats[j])


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def exact_gemm(A, B, sfA, sfB, block: int = 128):
    """Exact rational block-scaled NT product of small code matrices."""
    M, K = A.shape
    N = B.shape[0]
    KB = K // block
    out = [[Fraction(0)] * N for _ in range(M)]
    a = [[fp8_fraction(int(c)) for c in row] for row in A]
    b = [[fp8_fraction(int(c)) for c in row] for row in B]
    for m in range(M):
        for n in range(N):
            total = Fraction(0)
            for kb in range(KB):
                s = Fraction(0)
                for k in range(kb * block, (kb + 1) * block):
                    s += a[m][k] * b[n][k]
                total += s * Fraction(float(sfA[m, kb])) * Fraction(float(sfB[n // block, kb]))
            out[m][n] = total
    return out
