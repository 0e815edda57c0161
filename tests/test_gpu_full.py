"""GPU parity at the full workload shapes, every output compared with the oracle.

The prefill GEMM (4096x7168x18432), the contiguous MoE workload (32 experts, N=4096,
K=7168, 8192 Zipf-routed tokens) and the masked MoE workload (32 x 256 rows, N=7168,
K=2048) run in the launch configuration the benchmark times; each is checked
* on seeded N(0,1) inputs: every produced output within the tolerance, and within
  the error model of the two-level accumulation (tests/parity.py, MFMA_EPS);
* on integer-valued inputs at the same shapes (codes decoding to integers in [-8, 8],
  unit or power-of-two scales): every partial sum is an exact fp32 integer, so every
  output must equal the oracle's bf16 rounding bit for bit;
* for the grouped layouts, rows that are not produced keep their seeded sentinel
  bytes and the 64 KB guard bands around C stay intact.
The result a produced output must match is the plain block-scaled product of the
DeepGEMM launch article (deepseek.csdn.net), section 1.2 "precision safeguards".
"""
import time

import numpy as np
import pytest

import oracle
import synth
from tests import parity
from tests.parity import assert_bitwise, assert_parity, abs_product_sum, error_model_report
from tests.test_gpu_parity import INT_CODES, run_contiguous, run_dense, run_masked

pytestmark = [pytest.mark.gpu, pytest.mark.timeout(900)]


def _log(what, t0, **kv):
    print(f"[full] {what}: {time.perf_counter() - t0:.1f} s " +
          " ".join(f"{k}={v}" for k, v in kv.items()), flush=True)


def _check_model(g, r, ra, what):
    rep = error_model_report(g, r, ra)
    print(f"[full] {what} error model: {rep}", flush=True)
    assert rep["max_ratio"] <= parity.MFMA_EPS, f"{what}: beyond the MFMA error model {rep}"
    return rep


def int_codes(rng, shape):
    return rng.choice(INT_CODES, size=shape).astype(np.uint8)


# ------------------------------------------------------------------ dense prefill


def test_prefill_full():
    t0 = time.perf_counter()
    w = synth.workload("prefill")
    g = run_dense(w.A, w.B, w.sfA, w.sfB)
    _log("prefill gpu", t0)
    r = oracle.gemm_nt(w.A, w.B, w.sfA, w.sfB)
    _log("prefill oracle", t0)
    rep = assert_parity(g, r, what="prefill")
    print("[full] prefill:", rep, flush=True)
    ra = abs_product_sum(w.A, w.B, w.sfA, w.sfB)
    _log("prefill R_abs", t0)
    _check_model(g, r, ra, "prefill")


def test_prefill_integer_exact_full_bitwise():
    t0 = time.perf_counter()
    M, N, K = 4096, 7168, 18432
    rng = np.random.default_rng(4096)
    A = int_codes(rng, (M, K))
    B = int_codes(rng, (N, K))
    sfA = np.ones((M, K // 128), dtype=np.float32)
    sfB = np.ones((N // 128, K // 128), dtype=np.float32)
    g = run_dense(A, B, sfA, sfB)
    _log("prefill int gpu", t0)
    assert_bitwise(g, oracle.gemm_nt(A, B, sfA, sfB), "prefill integer-exact")
    _log("prefill int oracle", t0)


# ------------------------------------------------------------------ contiguous


def _contiguous_checks(w, g, init, exact):
    r, produced = oracle.grouped_contiguous(w.A, w.B, w.sfA, w.sfB, w.m_indices)
    assert np.array_equal(g[~produced], init[~produced]), "pad rows touched"
    assert produced.sum() == (w.m_indices >= 0).sum()
    if exact:
        assert_bitwise(g[produced], r[produced], "contiguous integer-exact")
        return r, produced
    rep = assert_parity(g[produced], r[produced], what="contiguous")
    print("[full] moe_cont:", rep, flush=True)
    return r, produced


def _contiguous_abs(w, produced):
    ra = np.zeros((w.A.shape[0], w.B.shape[1]))
    for e in range(w.B.shape[0]):
        rows = np.nonzero(w.m_indices == e)[0]
        if rows.size:
            ra[rows] = abs_product_sum(w.A[rows], w.B[e], w.sfA[rows], w.sfB[e])
    return ra


def test_contiguous_workload_full():
    t0 = time.perf_counter()
    w = synth.workload("moe_cont")
    g, init = run_contiguous(w.A, w.B, w.sfA, w.sfB, w.m_indices)
    _log("moe_cont gpu", t0)
    r, produced = _contiguous_checks(w, g, init, exact=False)
    _log("moe_cont oracle", t0)
    ra = _contiguous_abs(w, produced)
    _check_model(g[produced], r[produced], ra[produced], "moe_cont")


def test_contiguous_integer_exact_full_bitwise():
    """The real routing (8192 Zipf(1.1) tokens over 28 of 32 experts, 128-aligned
    segments, pad rows -1) with integer-valued operands and power-of-two scales."""
    t0 = time.perf_counter()
    lay = synth.workload("moe_cont")
    M_total, N, K, G = lay.shape
    rng = np.random.default_rng(9856)

    class W:
        pass

    w = W()
    w.m_indices = lay.m_indices
    w.A = int_codes(rng, (M_total, K))
    w.B = int_codes(rng, (G, N, K))
    w.sfA = np.ldexp(1.0, rng.integers(-1, 2, size=(M_total, K // 128))).astype(np.float32)
    w.sfB = np.ldexp(1.0, rng.integers(-1, 2, size=(G, N // 128, K // 128))).astype(np.float32)
    g, init = run_contiguous(w.A, w.B, w.sfA, w.sfB, w.m_indices)
    _log("moe_cont int gpu", t0)
    _contiguous_checks(w, g, init, exact=True)
    _log("moe_cont int oracle", t0)


# ------------------------------------------------------------------ masked


def _masked_checks(w, g, init, exact):
    r, produced = oracle.grouped_masked(w.A, w.B, w.sfA, w.sfB, w.masked_m)
    assert np.array_equal(g[~produced], init[~produced]), "masked rows touched"
    if exact:
        assert_bitwise(g[produced], r[produced], "masked integer-exact")
        return r, produced
    rep = assert_parity(g[produced], r[produced], what="masked")
    print("[full] moe_mask:", rep, flush=True)
    return r, produced


def test_masked_workload_full():
    t0 = time.perf_counter()
    w = synth.workload("moe_mask", pad_code=synth.FP8_NAN_CODE)
    g, init = run_masked(w.A, w.B, w.sfA, w.sfB, w.masked_m, int(w.masked_m.mean()))
    _log("moe_mask gpu", t0)
    r, produced = _masked_checks(w, g, init, exact=False)
    _log("moe_mask oracle", t0)
    G, M_max, N, K = w.shape
    ra = np.zeros((G, M_max, N))
    for e in range(G):
        v = int(w.masked_m[e])
        if v > 0:
            ra[e, :v] = abs_product_sum(w.A[e, :v], w.B[e], w.sfA[e, :v], w.sfB[e])
    _check_model(g[produced], r[produced], ra[produced], "moe_mask")


def test_masked_integer_exact_full_bitwise():
    """The real masked draw (32 experts, masked_m uniform on 0..256) with integer-valued
    operands; masked rows hold the NaN code, which must never reach an output."""
    t0 = time.perf_counter()
    lay = synth.workload("moe_mask")
    G, M_max, N, K = lay.shape
    rng = np.random.default_rng(7168)

    class W:
        pass

    w = W()
    w.masked_m = lay.masked_m
    w.A = int_codes(rng, (G, M_max, K))
    for e in range(G):
        w.A[e, max(int(w.masked_m[e]), 0):] = synth.FP8_NAN_CODE
    w.B = int_codes(rng, (G, N, K))
    w.sfA = np.ldexp(1.0, rng.integers(-1, 2, size=(G, M_max, K // 128))).astype(np.float32)
    w.sfB = np.ldexp(1.0, rng.integers(-1, 2, size=(G, N // 128, K // 128))).astype(np.float32)
    g, init = run_masked(w.A, w.B, w.sfA, w.sfB, w.masked_m, int(w.masked_m.mean()))
    _log("moe_mask int gpu", t0)
    _masked_checks(w, g, init, exact=True)
    _log("moe_mask int oracle", t0)
