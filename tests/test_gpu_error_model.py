"""The error model of the two-level accumulation on gfx950, measured through the C ABI.

The DeepGEMM launch article (deepseek.csdn.net), section 1.2 "precision safeguards",
promotes the FP8 products to FP32 once per block because the matrix instruction does
not keep a full-precision running sum. These tests measure what the gfx950 FP8 MFMA
keeps of its own internal sum, on inputs whose exact result is known:

* cancellation probes: in one 128-wide K-block a product +P and a product -P cancel
  exactly, and one small product q is added; the exact result is q (a power of two,
  exact in bf16). Whether q survives, for q/P from 2^-9 down to 2^-27, shows how many
  bits below the largest product of an accumulation group the hardware keeps;
* group probes: which K positions share an accumulation group (8 consecutive ones,
  8-aligned, for every instruction shape the kernels use);
* the bound tests/parity.py states (|g - r| <= ulp/2 + MFMA_EPS * R_abs) on N(0,1)
  inputs across the kernel families.
"""
import numpy as np
import pytest

import oracle
import synth
from tests import gpu_util as gu
from tests import parity
from tests.parity import abs_product_sum, error_model_report
from tests.test_gpu_parity import run_dense

pytestmark = pytest.mark.gpu


def pow2_code(j: int) -> int:
    """e4m3fn code of 2^-j, j in 0..9."""
    assert 0 <= j <= 9
    if j <= 6:
        return (7 - j) << 3
    return {7: 0x04, 8: 0x02, 9: 0x01}[j]


def cancellation_operands(M, N, p0, p1, p2):
    """A row m: +448 at p0, -448 at p1, 2^-(m % 10) at p2; B row n: 1 at p0 and p1,
    2^-(n % 10) at p2 (and 448 for n >= 10, so the small product also spans upward).
    Exact C[m][n] = 2^-(m%10) * b(n, p2)."""
    K = 128
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    A[:, p0] = 0x7E
    A[:, p1] = 0xFE
    for m in range(M):
        A[m, p2] = pow2_code(m % 10)
    B[:, p0] = 0x38
    B[:, p1] = 0x38
    for n in range(N):
        B[n, p2] = pow2_code(n % 10)
    return A, B


CONFIGS = ["pipe128x256", "stream_w4_tn1_d10", "skinny_w4_tn1_d2", "tile64x64_w2x2"]


def _rows(cfg):
    return 128 if cfg.startswith("pipe") or cfg.startswith("tile") else 64


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("pos,same_group", [((0, 1, 2), True), ((5, 70, 6), True),
                                            ((0, 64, 127), False), ((127, 0, 64), False)])
def test_cancellation_probe(cfg, pos, same_group, monkeypatch):
    """+448 at p0, -448 at p1, q at p2 (all in one K-block), exact result q.
    When q shares its group with the 448 product (p2 next to p0), q survives exactly
    when q >= 2^(8-13) (448 lies in [2^8, 2^9)) and vanishes when q <= 2^(8-14).
    When q sits in a group of its own and p0, p1 in others, the group sums meet at
    fp32 resolution: q survives down to 2^-15 (one fp32 ulp of 448) when the two
    large products are in different groups, and at every size when they cancel
    inside one group."""
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    M, N = _rows(cfg), 32
    A, B = cancellation_operands(M, N, *pos)
    sfA = np.ones((M, 1), np.float32)
    sfB = np.ones((1, 1), np.float32)
    g = run_dense(A, B, sfA, sfB)
    r = oracle.gemm_nt(A, B, sfA, sfB)
    gv = parity.bf16_to_f64(g)
    q = np.abs(r)
    kept = gv == r
    lost = gv == 0.0
    summary = {float(np.log2(v)): (int(kept[q == v].sum()), int(lost[q == v].sum()))
               for v in np.unique(q)}
    print(f"\n[probe] {cfg} pos={pos}: log2 q -> (kept, lost): {summary}", flush=True)
    assert np.all(kept | lost), "a result that is neither q nor 0"
    if same_group:
        assert np.all(kept[q >= 2.0 ** -5]) and np.all(lost[q <= 2.0 ** -6])
    elif pos == (0, 64, 127):
        assert np.all(kept)
    else:
        assert np.all(kept[q >= 2.0 ** -15]) and np.all(lost[q <= 2.0 ** -16])


@pytest.mark.parametrize("cfg", CONFIGS)
def test_group_membership_probe(cfg, monkeypatch):
    """Which K positions of a block share an accumulation group with position p0: row m
    holds 448 at p0 and 2^-9 at k = m in block 0, and -448 in block 1. The result is
    2^-9 when k = m lies outside p0's group (its group sum is exact, and fp32 resolves
    448 + 2^-9), 0 when inside (2^-9 is 17 binades below 448 in the same group)."""
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    M, N, K = 128, 16, 256
    if not cfg.startswith("pipe") and not cfg.startswith("tile"):
        M = 64  # the M <= 64 kernels; rows m cover k = 0..63, a second call k = 64..127
    groups = {}
    for p0 in (0, 3, 17, 40, 64, 77, 100, 127):
        members = []
        for base in range(0, 128, M):
            A = np.zeros((M, K), np.uint8)
            B = np.zeros((N, K), np.uint8)
            A[:, p0] = 0x7E
            A[:, 128] = 0xFE
            for m in range(M):
                if base + m != p0:
                    A[m, base + m] = 0x01
            B[:, :129] = 0x38
            g = parity.bf16_to_f64(run_dense(A, B, np.ones((M, 2), np.float32),
                                             np.ones((1, 2), np.float32)))
            assert np.all((g == 0.0) | (g == 2.0 ** -9))
            assert np.all(g == g[:, :1]), "columns disagree"
            members += [base + m for m in range(M) if g[m, 0] == 0.0]
        groups[p0] = frozenset(members)
        print(f"[group] {cfg} p0={p0}: {sorted(members)}", flush=True)
    # measured on gfx950: every instruction shape groups the 8 consecutive K positions
    # of an 8-aligned run (one group = products 8j .. 8j + 7 of the block)
    for p0, grp in groups.items():
        assert grp == frozenset(range(p0 // 8 * 8, p0 // 8 * 8 + 8)), (p0, sorted(grp))


@pytest.mark.parametrize("M,N,K,seed", [(128, 256, 512, 1), (64, 2112, 7168, 2),
                                        (64, 4096, 512, 3), (300, 528, 2048, 4),
                                        (256, 1280, 4096, 5)])
def test_error_model_gaussian(M, N, K, seed):
    w = synth.dense(M, N, K, seed_base=424000 + seed)
    g = run_dense(w.A, w.B, w.sfA, w.sfB)
    r = oracle.gemm_nt(w.A, w.B, w.sfA, w.sfB)
    rep = error_model_report(g, r, abs_product_sum(w.A, w.B, w.sfA, w.sfB))
    print(f"\n[model] {M}x{N}x{K}: {rep}", flush=True)
    assert rep["max_ratio"] <= parity.MFMA_EPS


def adversarial_operands(rng, M, N, K):
    """Groups built to be cut: per 8 consecutive K positions of each row of B one large
    code and seven small ones spread around 2^-13 of it (subnormals and small
    normals), against N(0,1)-like A codes."""
    A = rng.choice(np.array([0x30, 0x34, 0x38, 0x3C, 0x40, 0xB8, 0xC0, 0x44, 0xC4], np.uint8),
                   size=(M, K))
    small = np.array([0x01, 0x02, 0x03, 0x05, 0x07, 0x08, 0x0B, 0x10, 0x13, 0x18, 0x1D,
                      0x81, 0x86, 0x90, 0x98], np.uint8)
    B = rng.choice(small, size=(N, K))
    big = rng.integers(0, 8, size=(N, K // 8))
    for j in range(K // 8):
        B[np.arange(N), 8 * j + big[:, j]] = rng.choice(np.array([0x7E, 0x76, 0xFE, 0x6E], np.uint8), N)
    sfA = np.ldexp(1.0, rng.integers(-3, 4, size=(M, K // 128))).astype(np.float32)
    sfB = np.ldexp(1.0, rng.integers(-3, 4, size=((N + 127) // 128, K // 128))).astype(np.float32)
    return A.astype(np.uint8), B.astype(np.uint8), sfA, sfB


@pytest.mark.parametrize("cfg", CONFIGS)
@pytest.mark.parametrize("data", ["gaussian", "adversarial"])
def test_per_output_model_bound(cfg, data, monkeypatch):
    """Every output within ulp/2 of its fp32 value plus the model's per-output bound
    (tests/parity.py model_bound); on the adversarial inputs the cut products make
    the error far larger than on Gaussian data, and the bound still holds."""
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    M = _rows(cfg)
    N, K = 272, 1024
    rng = np.random.default_rng(len(cfg) * 31 + len(data))
    if data == "gaussian":
        w = synth.dense(M, N, K, seed_base=425000 + len(cfg))
        A, B, sfA, sfB = w.A, w.B, w.sfA, w.sfB
    else:
        A, B, sfA, sfB = adversarial_operands(rng, M, N, K)
    g = run_dense(A, B, sfA, sfB)
    r = oracle.gemm_nt(A, B, sfA, sfB)
    bound = parity.model_bound(A, B, sfA, sfB, k_roundings=K // 128 + 8)
    gv = parity.bf16_to_f64(g)
    hu = parity.half_ulp_bf16(np.abs(gv))
    over = np.abs(gv - r) - hu
    ratio = float(np.max(over / bound))
    rabs = abs_product_sum(A, B, sfA, sfB)
    flat = float(np.max(np.maximum(over, 0) / rabs))
    print(f"\n[bound] {cfg} {data}: max (|g-r| - ulp/2) / bound = {ratio:.3g}; "
          f"against R_abs {flat:.3g}", flush=True)
    assert ratio <= 1.0
