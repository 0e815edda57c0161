"""Parity gate between a bf16 GPU result and the oracle's fp64 value.

Tolerance (the stated bar is a maximum relative error of 2e-3 for bf16 output; the
pages give none). A literal elementwise |g - r| / |r| <= 2e-3 cannot hold even for
a perfectly rounded bf16 output (bf16 rounding alone reaches 2^-8 ~ 3.9e-3 relative,
and the ratio is unbounded near zero), so the bar is read as a bound on the kernel's
own error on top of the one unavoidable output rounding:

    |g - r| <= ulp_bf16(max(|r|, |g|)) / 2 + 2e-3 * max(|r|, rho / 16)

with r the oracle's fp64 value, g the GPU's bf16 value, rho the RMS of r over the
call's produced outputs, ulp_bf16(v) = 2^(floor(log2 v) - 7). Reported alongside:
the worst excess (|g - r| - ulp/2)+ / max(|r|, rho/16), the Frobenius relative
error, and the fraction of outputs bitwise equal to the oracle's bf16 rounding.
"""
from __future__ import annotations

import numpy as np

import oracle

REL_TOL = 2e-3

# Error model of the two-level accumulation on gfx950 (tests/test_gpu_error_model.py
# pins it). The FP8 matrix instruction sums its products in groups: inside a group the
# products are aligned to the largest one and bits more than 13 binades below it are
# dropped; the group sums are then added at fp32 resolution. Promotion across K-blocks
# and split-K sums add fp32 roundings of at most 2^-24 of the running magnitude.
# The error of the fp32 result before the output rounding is therefore a small
# multiple of 2^-13 of the products' magnitudes. Stated against
#     R_abs[m][n] = sum_k |sfA[m][k/128] * sfB[n/128][k/128] * a(m,k) * b(n,k)|,
# the parity tests assert, on the configured inputs (N(0,1) blocks quantized per
# 1x128 / 128x128 with power-of-two scales),
#     |g - r| <= ulp_bf16(max(|r|, |g|)) / 2 + MFMA_EPS * R_abs,   MFMA_EPS = 2^-16.
# The largest excess measured on such inputs, over every kernel family and the full
# workloads, is 5.2e-6 * R_abs (about 2^-17.6); an input that puts many products just
# under 2^-13 of a much larger one in the same group can exceed this bound (up to
# about group size * 2^-13), which is why it is stated for these inputs only.
MFMA_EPS = 2.0 ** -16


def bf16_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def half_ulp_bf16(v: np.ndarray) -> np.ndarray:
    v = np.maximum(np.abs(v), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(v)).astype(np.int64) - 8)


def report(g_bits, r_exact, rho: float | None = None) -> dict:
    g_bits = np.asarray(g_bits, dtype=np.uint16).ravel()
    r = np.asarray(r_exact, dtype=np.float64).ravel()
    g = bf16_to_f64(g_bits)
    if rho is None:
        rho = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    floor = max(rho / 16.0, 1e-300)
    denom = np.maximum(np.abs(r), floor)
    hu = half_ulp_bf16(np.maximum(np.abs(r), np.abs(g)))
    err = np.abs(g - r)
    excess = np.maximum(err - hu, 0.0) / denom
    ok = err <= hu + REL_TOL * denom
    ref_bits = oracle.bf16_rne(r)
    nr = np.linalg.norm(r)
    return {
        "n": int(r.size),
        "rho": rho,
        "max_excess_rel": float(excess.max()) if r.size else 0.0,
        "frobenius_rel": float(np.linalg.norm(g - r) / nr) if nr > 0 else float(np.linalg.norm(g)),
        "bitwise_match": float(np.mean(g_bits == ref_bits)) if r.size else 1.0,
        "n_fail": int((~ok).sum()),
        "nan": int(np.isnan(g).sum()),
        "worst_index": int(np.argmax(excess)) if r.size else -1,
    }


def abs_values() -> np.ndarray:
    """|value| of every e4m3fn code (0 for the NaN codes, which only pad rows hold)."""
    v = np.abs(oracle.e4m3fn_values())
    v[np.isnan(v)] = 0.0
    return v


def abs_product_sum(A, B, sfA, sfB) -> np.ndarray:
    """R_abs [M][N] = sum_k |sfA[m][kb] sfB[n/128][kb] a(m,k) b(n,k)|, kb = k / 128: the
    block-scaled product of the operands' absolute values, as one fp64 matrix product of
    the scaled magnitudes (every term is non-negative, so fp64 carries it to ~1e-12)."""
    import torch
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    M, K = A.shape
    N = B.shape[0]
    KB = K // 128
    vals = torch.from_numpy(abs_values())
    sa = torch.from_numpy(np.asarray(sfA, dtype=np.float32).astype(np.float64)).abs()
    sb = torch.from_numpy(np.asarray(sfB, dtype=np.float32).astype(np.float64)).abs()
    out = torch.empty((M, N), dtype=torch.float64)
    step = 1024  # rows of A per product, to bound the fp64 copies
    bh = vals[torch.from_numpy(B).long()].view(N, KB, 128)
    bh *= sb[torch.arange(N) // 128].view(N, KB, 1)
    bh = bh.view(N, K)
    for m0 in range(0, M, step):
        ah = vals[torch.from_numpy(A[m0:m0 + step]).long()].view(-1, KB, 128)
        ah *= sa[m0:m0 + step].view(-1, KB, 1)
        out[m0:m0 + step] = ah.view(-1, K) @ bh.T
    return out.numpy()


def model_bound(A, B, sfA, sfB, k_roundings: int) -> np.ndarray:
    """Per-output bound on |fp32 result - exact| from the probed FP8 MFMA mechanism:
    in each group of 8 consecutive K positions the products are aligned to the largest
    one, of exponent E, and kept to multiples of 2^(E-13), so a product loses at most
    its residue modulo 2^(E-13) (truncated or rounded); group sums, the block's
    promotion, the split-K sums and the accumulation across blocks are fp32 additions,
    each rounding by at most 2^-24 of a partial sum bounded by R_abs. Returns
        sum_kb sfA sfB sum_groups sum_k (|a b| mod 2^(E_g - 13))
        + (16 + k_roundings) * 2^-24 * R_abs
    for small shapes (a loop over groups on the host)."""
    vals = abs_values()
    A = np.asarray(A, dtype=np.uint8)
    B = np.asarray(B, dtype=np.uint8)
    M, K = A.shape
    N = B.shape[0]
    av, bv = vals[A], vals[B]
    sa = np.asarray(sfA, dtype=np.float64)
    sb = np.asarray(sfB, dtype=np.float64)[np.arange(N) // 128]
    trunc = np.zeros((M, N))
    for g0 in range(0, K, 8):
        kb = g0 // 128
        P = av[:, None, g0:g0 + 8] * bv[None, :, g0:g0 + 8]  # exact in fp64
        pmax = P.max(axis=2)
        E = np.floor(np.log2(np.where(pmax > 0, pmax, 1.0)))
        q = np.ldexp(1.0, (E - 13).astype(np.int64))
        res = np.fmod(P, q[:, :, None]).sum(axis=2)
        trunc += np.where(pmax > 0, res, 0.0) * sa[:, kb, None] * sb[None, :, kb]
    return trunc + (16 + k_roundings) * 2.0 ** -24 * abs_product_sum(A, B, sfA, sfB)


def error_model_report(g_bits, r_exact, r_abs) -> dict:
    """How far each output is from the exact value beyond the output rounding, as a
    fraction of its absolute-product sum: max over outputs of
    (|g - r| - ulp_bf16(max(|r|,|g|))/2)+ / R_abs, and the worst ulp distance from the
    oracle's own bf16 rounding."""
    g_bits = np.asarray(g_bits, dtype=np.uint16).ravel()
    r = np.asarray(r_exact, dtype=np.float64).ravel()
    ra = np.asarray(r_abs, dtype=np.float64).ravel()
    g = bf16_to_f64(g_bits)
    hu = half_ulp_bf16(np.maximum(np.abs(r), np.abs(g)))
    over = np.maximum(np.abs(g - r) - hu, 0.0)
    ratio = np.where(ra > 0, over / np.maximum(ra, 1e-300), np.where(over > 0, np.inf, 0.0))
    ref = oracle.bf16_rne(r).astype(np.int64)
    gi = g_bits.astype(np.int64)
    # ulp distance between two bf16 patterns: order them as integers on one line
    key = lambda b: np.where(b & 0x8000, -(b & 0x7FFF), b)
    ulps = np.abs(key(gi) - key(ref))
    return {"max_ratio": float(ratio.max()) if r.size else 0.0,
            "max_ulps": int(ulps.max()) if r.size else 0,
            "n_off_by_more_than_1ulp": int((ulps > 1).sum()),
            "n_mismatch": int((ulps > 0).sum())}


def assert_error_model(g_bits, r_exact, r_abs, what: str = "") -> dict:
    rep = error_model_report(g_bits, r_exact, r_abs)
    assert rep["max_ratio"] <= MFMA_EPS, (f"{what}: error beyond the MFMA model "
                                          f"({rep['max_ratio']:.3g} > {MFMA_EPS:.3g}) {rep}")
    return rep


def assert_parity(g_bits, r_exact, rho: float | None = None, what: str = "") -> dict:
    rep = report(g_bits, r_exact, rho)
    assert rep["nan"] == 0, f"{what}: NaN in GPU output {rep}"
    assert rep["n_fail"] == 0, f"{what}: {rep['n_fail']} outputs beyond tolerance {rep}"
    return rep


def assert_bitwise(g_bits, r_exact, what: str = "") -> None:
    ref = oracle.bf16_rne(np.asarray(r_exact, dtype=np.float64))
    g = np.asarray(g_bits, dtype=np.uint16)
    bad = np.nonzero(g.ravel() != ref.ravel())[0]
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} differ bitwise; first at flat "
                           f"{bad[0]}: gpu {g.ravel()[bad[0]]:#06x} oracle {ref.ravel()[bad[0]]:#06x}")
