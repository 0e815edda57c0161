"""CPU checks of the seeded input generator (synth/): its engine, distributions and
layouts, and that its fast quantizer agrees code for code with the oracle's
search-based quantizer."""
import numpy as np
import pytest

import oracle
import synth


def test_mt19937_64_standard_value():
    # the C++ standard fixes the 10000th output of a default-seeded mt19937_64
    assert synth.mt_output(5489, 10000) == 9981545732273789042


def test_normals_moments_and_determinism():
    x = synth.normal_rows(77, 600, 1024)
    assert abs(x.mean()) < 0.01 and abs(x.std() - 1) < 0.01
    assert np.array_equal(x, synth.normal_rows(77, 600, 1024))
    # chunks of 128 rows are independent streams: a shorter draw is a prefix
    assert np.array_equal(synth.normal_rows(77, 130, 1024), x[:130])


@pytest.mark.parametrize("br", [1, 128])
def test_make_operand_equals_draw_then_quantize(br):
    R, C = 300, 512
    codes, sf = synth.make_operand(91, R, C, br)
    x = synth.normal_rows(91, R, C)
    c2, s2 = synth.quantize(x, br)
    assert np.array_equal(codes, c2) and np.array_equal(sf, s2)


@pytest.mark.parametrize("br", [1, 128])
def test_fast_quantizer_matches_oracle(br):
    rng = np.random.default_rng(5)
    R, C = 260, 384
    x = (rng.standard_normal((R, C)) * rng.lognormal(0, 8, (R, 1))).astype(np.float32)
    x[3, :128] = 0.0
    x[4, :128] = -0.0
    x[5, 5] = np.float32(1e-30)
    c1, s1 = synth.quantize(x, br)
    c2, s2 = oracle.quantize_blocks(x, br, 128)
    assert np.array_equal(s1, s2)
    assert np.array_equal(c1, c2)


def test_fast_quantizer_matches_oracle_on_every_midpoint():
    vals = oracle.e4m3fn_values()[:127]
    ys = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2]).astype(np.float32).astype(np.float64)
    ys = np.concatenate([ys, np.nextafter(ys, np.inf), np.nextafter(ys, -np.inf)])
    ys = ys[(ys >= 0) & (ys <= 448)]
    ys = np.concatenate([ys, -ys]).astype(np.float32)
    n = (ys.size // 128) * 128
    x = ys[:n].reshape(-1, 128).copy()
    x[:, 0] = 448.0  # pin each block's scale to 1 so the probes are coded as they are
    c1, s1 = synth.quantize(x, 1)
    c2, s2 = oracle.quantize_blocks(x, 1, 128)
    assert np.all(s1 == 1.0) and np.array_equal(c1, c2)


def test_contiguous_layout_rules():
    w = synth.workload("moe_cont")
    M_total, N, K, G = w.shape
    assert (G, N, K) == (32, 4096, 7168)
    assert int(w.counts.sum()) == 8192
    assert int((w.counts == 0).sum()) == 4
    assert M_total % 128 == 0
    mi = w.m_indices
    groups = mi.reshape(-1, 128)
    for g in groups:
        ids = set(g[g >= 0].tolist())
        assert len(ids) == 1  # every 128-row group holds exactly one expert
    # segments in expert-id order, real rows first, then pad
    real = mi[mi >= 0]
    assert np.all(np.diff(real) >= 0)
    for e in range(G):
        assert int((mi == e).sum()) == int(w.counts[e])
    # pad rows: code 0, scale 1
    assert np.all(w.A[mi < 0] == 0) and np.all(w.sfA[mi < 0] == 1.0)


def test_zipf_is_skewed_and_permutation_valid():
    c = synth.zipf_counts(4003, 8192, 28, 1.1)
    assert c.sum() == 8192 and c[0] > c[5] > c[27]
    p = synth.permutation(4004, 32)
    assert sorted(p.tolist()) == list(range(32))


def test_masked_counts_in_range():
    m = synth.uniform_ints(5003, 10000, 257)
    assert m.min() == 0 and m.max() == 256
    w = synth.masked(4, 64, 256, 256, 9000)
    assert np.all((w.masked_m >= 0) & (w.masked_m <= 64))
    for e in range(4):
        assert np.all(w.A[e, w.masked_m[e]:] == 0)
