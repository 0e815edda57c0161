"""CPU pins for the oracle's block-scaled GEMM (dense, contiguous, masked).

Pins, each independent of the oracle's own arithmetic:
  * a hand-worked example (tests/golden/hand_dense_2x3x256.txt);
  * exact rational brute force on tiny shapes (Python Fractions over torch-decoded
    fp8 values), with power-of-two scales (must be exact) and arbitrary scales;
  * closed forms: identity B, one-hot A rows, constant matrices;
  * exact doubling when one scale row or block is doubled;
  * grouped layouts equal per-expert dense products, pad / masked rows not produced.
A plausible slip (a dropped block, a sign, the sfB index n/128, a transposed operand,
a wrong expert offset) fails at least one of these.
"""
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from tests import _exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
VALS = _exact.fp8_values_torch()
FINITE = np.array([c for c in range(256) if not np.isnan(VALS[c])], dtype=np.uint8)


def rand_codes(rng, shape):
    return rng.choice(FINITE, size=shape).astype(np.uint8)


def pow2_scales(rng, shape, lo=-6, hi=6):
    return np.ldexp(1.0, rng.integers(lo, hi + 1, size=shape)).astype(np.float32)


def _runs(tokens):
    out = []
    for t in tokens:
        cnt, code = t.split(":")
        out += [int(code, 16)] * int(cnt)
    return out


def load_hand_example():
    d = {"A": [], "B": [], "sfA": [], "sfB": [], "C": [], "Cbf16": []}
    with open(os.path.join(GOLDEN, "hand_dense_2x3x256.txt")) as f:
        for ln in f:
            if not ln.strip() or ln.startswith("#"):
                continue
            key, *rest = ln.split()
            if key in ("M", "N", "K"):
                d[key] = int(rest[0])
            elif key in ("A", "B"):
                d[key].append(_runs(rest))
            elif key == "Cbf16":
                d[key].append([int(v, 16) for v in rest])
            else:
                d[key].append([float(v) for v in rest])
    return d


def test_hand_worked_example():
    d = load_hand_example()
    A = np.array(d["A"], dtype=np.uint8)
    B = np.array(d["B"], dtype=np.uint8)
    assert A.shape == (d["M"], d["K"]) and B.shape == (d["N"], d["K"])
    C = oracle.gemm_nt(A, B, np.array(d["sfA"]), np.array(d["sfB"]))
    assert np.array_equal(C, np.array(d["C"]))
    assert np.array_equal(oracle.bf16_rne(C), np.array(d["Cbf16"], dtype=np.uint16))


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (2, 3, 256), (3, 17, 128), (4, 130, 128),
                                   (17, 2, 256)])
def test_dense_exact_rational_pow2_scales(M, N, K):
    rng = np.random.default_rng(M * 1000 + N * 10 + K)
    A, B = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sfA = pow2_scales(rng, (M, K // 128))
    sfB = pow2_scales(rng, ((N + 127) // 128, K // 128))
    C = oracle.gemm_nt(A, B, sfA, sfB)
    ex = _exact.exact_gemm(A, B, sfA, sfB)
    ref = oracle.bf16_rne(C)
    for m in range(M):
        for n in range(N):
            # with power-of-two scales and K <= 256 the fp64 sum is exact
            assert Fraction(float(C[m, n])) == ex[m][n]
            assert int(ref[m, n]) == _exact.bf16_round_exact(ex[m][n]) or ex[m][n] == 0


def test_dense_exact_rational_arbitrary_scales():
    # non-power-of-two scales: the scaled block terms and their fp64 sum round, by at
    # most a few fp64 ulps of the sum of |terms|
    rng = np.random.default_rng(5)
    M, N, K = 3, 5, 384
    A, B = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sfA = rng.uniform(0.01, 3.0, (M, 3)).astype(np.float32)
    sfB = rng.uniform(0.01, 3.0, (1, 3)).astype(np.float32)
    C = oracle.gemm_nt(A, B, sfA, sfB)
    ex = _exact.exact_gemm(A, B, sfA, sfB)
    for m in range(M):
        for n in range(N):
            abs_terms = Fraction(0)
            for kb in range(3):
                blk = _exact.exact_gemm(A[m:m + 1, kb * 128:(kb + 1) * 128],
                                        B[n:n + 1, kb * 128:(kb + 1) * 128],
                                        sfA[m:m + 1, kb:kb + 1], sfB[:, kb:kb + 1])[0][0]
                abs_terms += abs(blk)
            assert abs(Fraction(float(C[m, n])) - ex[m][n]) <= 8 * Fraction(2) ** -53 * abs_terms


def test_identity_B():
    rng = np.random.default_rng(21)
    M, K = 7, 256
    A = rand_codes(rng, (M, K))
    sfA = pow2_scales(rng, (M, 2))
    B = np.zeros((K, K), dtype=np.uint8)
    B[np.arange(K), np.arange(K)] = 0x38  # 1.0 on the diagonal
    sfB = np.ones((2, 2), dtype=np.float32)
    C = oracle.gemm_nt(A, B, sfA, sfB)
    want = VALS[A] * np.repeat(sfA, 128, axis=1)
    assert np.array_equal(C, want)


def test_one_hot_rows():
    rng = np.random.default_rng(22)
    M, N, K = 4, 200, 384
    B = rand_codes(rng, (N, K))
    sfB = pow2_scales(rng, (2, 3))
    A = np.zeros((M, K), dtype=np.uint8)
    ks = [0, 127, 128, 383]
    codes = [0x38, 0xC4, 0x01, 0x7E]
    for m, (k, c) in enumerate(zip(ks, codes)):
        A[m, k] = c
    sfA = pow2_scales(rng, (M, 3))
    C = oracle.gemm_nt(A, B, sfA, sfB)
    for m, (k, c) in enumerate(zip(ks, codes)):
        kb = k // 128
        want = VALS[c] * VALS[B[:, k]] * sfA[m, kb] * sfB[np.arange(N) // 128, kb]
        assert np.array_equal(C[m], want)


def test_constant_matrices_closed_form():
    M, N, K = 3, 260, 640
    A = np.full((M, K), 0x40, dtype=np.uint8)   # 2
    B = np.full((N, K), 0xB0, dtype=np.uint8)   # -0.5
    sfA = np.full((M, 5), 0.25, dtype=np.float32)
    sfB = np.full((3, 5), 8.0, dtype=np.float32)
    C = oracle.gemm_nt(A, B, sfA, sfB)
    assert np.all(C == 2 * -0.5 * K * 0.25 * 8.0)


def test_scale_doubling_is_exact():
    rng = np.random.default_rng(23)
    M, N, K = 5, 300, 512
    A, B = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sfA, sfB = pow2_scales(rng, (M, 4)), pow2_scales(rng, (3, 4))
    C = oracle.gemm_nt(A, B, sfA, sfB)
    sfA2 = sfA.copy()
    sfA2[2] *= 2
    C2 = oracle.gemm_nt(A, B, sfA2, sfB)
    assert np.array_equal(C2[2], 2 * C[2])
    assert np.array_equal(np.delete(C2, 2, 0), np.delete(C, 2, 0))
    sfB2 = sfB.copy()
    sfB2[1] *= 2  # columns 128..255 double, the rest unchanged
    C3 = oracle.gemm_nt(A, B, sfA, sfB2)
    assert np.array_equal(C3[:, 128:256], 2 * C[:, 128:256])
    assert np.array_equal(C3[:, :128], C[:, :128]) and np.array_equal(C3[:, 256:], C[:, 256:])
    # doubling one block's scale adds exactly that block's term
    sfA4 = sfA.copy()
    sfA4[1, 3] *= 2
    C4 = oracle.gemm_nt(A, B, sfA4, sfB)
    Ab = np.zeros_like(A)
    Ab[:, 384:512] = A[:, 384:512]
    term = oracle.gemm_nt(Ab, B, sfA, sfB)
    ex_new = _exact.exact_gemm(A[1:2], B[:4], sfA4[1:2], sfB)
    for n in range(4):
        assert Fraction(float(C4[1, n])) == ex_new[0][n]
        assert Fraction(float(C4[1, n])) == Fraction(float(C[1, n])) + Fraction(float(term[1, n]))


def test_gemm_at_matches_full():
    rng = np.random.default_rng(24)
    M, N, K = 9, 300, 384
    A, B = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sfA, sfB = pow2_scales(rng, (M, 3)), pow2_scales(rng, (3, 3))
    C = oracle.gemm_nt(A, B, sfA, sfB)
    mi = rng.integers(0, M, 500)
    ni = rng.integers(0, N, 500)
    assert np.array_equal(oracle.gemm_nt_at(A, B, sfA, sfB, mi, ni), C[mi, ni])


def test_contiguous_equals_per_expert_dense():
    rng = np.random.default_rng(25)
    G, N, K = 4, 200, 256
    m_indices = np.array([2] * 100 + [-1] * 28 + [0] * 128 + [3] * 5 + [-1] * 123 + [7] * 3 +
                         [-5] * 1 + [-1] * 124, dtype=np.int32)  # 7 and -5: out of range
    M_total = m_indices.size
    A = rand_codes(rng, (M_total, K))
    sfA = pow2_scales(rng, (M_total, 2))
    B = rand_codes(rng, (G, N, K))
    sfB = pow2_scales(rng, (G, 2, 2))
    C, produced = oracle.grouped_contiguous(A, B, sfA, sfB, m_indices)
    assert np.array_equal(produced, (m_indices >= 0) & (m_indices < G))
    assert np.all(np.isnan(C[~produced]))
    for e in range(G):
        rows = np.nonzero(m_indices == e)[0]
        if rows.size == 0:
            continue
        dense = oracle.gemm_nt(A[rows], B[e], sfA[rows], sfB[e])
        assert np.array_equal(C[rows], dense)
    ri = np.nonzero(produced)[0][rng.integers(0, produced.sum(), 300)]
    ni = rng.integers(0, N, 300)
    assert np.array_equal(oracle.grouped_contiguous_at(A, B, sfA, sfB, m_indices, ri, ni),
                          C[ri, ni])


def test_masked_equals_per_expert_dense():
    rng = np.random.default_rng(26)
    G, M_max, N, K = 5, 40, 130, 256
    masked_m = np.array([0, 40, 17, 99, -3], dtype=np.int32)  # 99 and -3 get clamped
    A = rand_codes(rng, (G, M_max, K))
    sfA = pow2_scales(rng, (G, M_max, 2))
    B = rand_codes(rng, (G, N, K))
    sfB = pow2_scales(rng, (G, 2, 2))
    C, produced = oracle.grouped_masked(A, B, sfA, sfB, masked_m)
    valid = np.clip(masked_m, 0, M_max)
    assert np.array_equal(produced, np.arange(M_max)[None, :] < valid[:, None])
    assert np.all(np.isnan(C[~produced]))
    for e in range(G):
        v = valid[e]
        if v == 0:
            continue
        assert np.array_equal(C[e, :v], oracle.gemm_nt(A[e, :v], B[e], sfA[e, :v], sfB[e]))
    ei = np.array([1, 2, 3, 1, 0])
    mi = np.array([39, 16, 39, 0, 0])
    ni = np.array([129, 0, 64, 5, 5])
    got = oracle.grouped_masked_at(A, B, sfA, sfB, masked_m, ei, mi, ni)
    assert np.array_equal(got[:4], C[ei[:4], mi[:4], ni[:4]]) and np.isnan(got[4])


def test_grouped_hand_example_rows():
    d = load_hand_example()
    A = np.array(d["A"], dtype=np.uint8)
    B = np.array(d["B"], dtype=np.uint8)[None]
    sfA = np.array(d["sfA"], dtype=np.float32)
    sfB = np.array(d["sfB"], dtype=np.float32)[None]
    C, produced = oracle.grouped_contiguous(A, B, sfA, sfB, np.array([0, -1], dtype=np.int32))
    assert produced.tolist() == [True, False]
    assert np.array_equal(C[0], np.array(d["C"][0]))
    Cm, pm = oracle.grouped_masked(A[None], B, sfA[None], sfB, np.array([2], dtype=np.int32))
    assert np.array_equal(Cm[0], np.array(d["C"]))


@pytest.mark.parametrize("layout", ["nt", "nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (3, 17, 256), (4, 130, 128)])
def test_layouts_exact_rational(layout, M, N, K):
    # op(A) op(B) with A stored [K][M] for "t" and B stored [K][N] for "n": against the
    # exact-rational NT product of transposed copies
    rng = np.random.default_rng(M * 7 + N + K + ord(layout[0]) + 3 * ord(layout[1]))
    A_mk, B_nk = rand_codes(rng, (M, K)), rand_codes(rng, (N, K))
    sfA = pow2_scales(rng, (M, K // 128))
    sfB = pow2_scales(rng, ((N + 127) // 128, K // 128))
    A = np.ascontiguousarray(A_mk.T) if layout[0] == "t" else A_mk
    B = np.ascontiguousarray(B_nk.T) if layout[1] == "n" else B_nk
    C = oracle.gemm(A, B, sfA, sfB, layout)
    ex = _exact.exact_gemm(A_mk, B_nk, sfA, sfB)
    for m in range(M):
        for n in range(N):
            assert Fraction(float(C[m, n])) == ex[m][n]
    assert np.array_equal(C, oracle.gemm_nt(A_mk, B_nk, sfA, sfB))
