"""GPU parity: the HIP library (through its C ABI, via the binding) against the CPU
oracle, element by element on the same seeded inputs.

* small shapes and edge shapes: every output compared;
* integer-exact inputs (codes decoding to small integers, power-of-two scales):
  every block partial and every accumulation step is exact in fp32, so the GPU must
  equal the oracle's bf16 rounding bitwise -- this pins all indexing;
* the full workload shapes: the decode shapes here, prefill and the MoE
  workloads in tests/test_gpu_full.py, every output in both;
* rows a grouped call must not produce keep their seeded sentinel bytes, and 64 KB
  guard bands around every output stay intact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu
from tests.parity import abs_product_sum, assert_bitwise, assert_error_model, assert_parity, report

pytestmark = pytest.mark.gpu

INT_CODES = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0x4A, 0x4C, 0x4E, 0x50,  # 0,1,2,3,4,5,6,7,8
                      0xB8, 0xC0, 0xC4, 0xC8, 0xCA, 0xCC, 0xCE, 0xD0], dtype=np.uint8)


def dg():
    import fp8_block_scaled_dg_amd as m
    return m


def int_operands(rng, M, N, K, G=None):
    KB, NB = K // 128, (N + 127) // 128
    shape_b = (N, K) if G is None else (G, N, K)
    A = rng.choice(INT_CODES, size=(M, K))
    B = rng.choice(INT_CODES, size=shape_b)
    sfA = np.ldexp(1.0, rng.integers(-2, 3, size=(M, KB))).astype(np.float32)
    sfB = np.ldexp(1.0, rng.integers(-2, 3, size=(NB, KB) if G is None else (G, NB, KB)))
    return A.astype(np.uint8), B.astype(np.uint8), sfA, sfB.astype(np.float32)


def run_dense(A, B, sfA, sfB, seed=1):
    M, K = A.shape
    N = B.shape[0]
    out = gu.Guarded((M, N), seed)
    gu.announce(f"dense M={M} N={N} K={K}")
    dg().fp8_gemm_nt(gu.codes(A), gu.codes(B), out.out, gu.dev(sfA), gu.dev(sfB))
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside C"
    return out.result()


# ------------------------------------------------------------------ dense


def test_dense_small_workload_full():
    w = synth.workload("small")
    g = run_dense(w.A, w.B, w.sfA, w.sfB)
    r = oracle.gemm_nt(w.A, w.B, w.sfA, w.sfB)
    rep = assert_parity(g, r, what="small")
    print("small:", rep)
    assert rep["bitwise_match"] > 0.98


@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (63, 64, 256), (64, 2112, 128), (65, 144, 384),
                                   (129, 272, 256), (200, 384, 512), (257, 128, 1024),
                                   (128, 256, 512)])
def test_dense_integer_exact_bitwise(M, N, K):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    A, B, sfA, sfB = int_operands(rng, M, N, K)
    g = run_dense(A, B, sfA, sfB)
    assert_bitwise(g, oracle.gemm_nt(A, B, sfA, sfB), what=f"int {M}x{N}x{K}")


# Tile counts that leave a partial last round on 256 CUs, with K long enough that the
# compute-bound kernel splits the tail tiles into 2, 4 and 8 K parts (whose partials
# are added by the last part to arrive). Integer-valued inputs keep every partial sum
# exact, so the split must not change a single bit.
@pytest.mark.parametrize("M,N,K", [(384, 768, 2048), (256, 1280, 4096), (128, 512, 8192),
                                   (300, 704, 3072)])
def test_dense_tail_split_integer_exact_bitwise(M, N, K):
    rng = np.random.default_rng(M * 5 + N + K * 3)
    A, B, sfA, sfB = int_operands(rng, M, N, K)
    g = run_dense(A, B, sfA, sfB)
    assert_bitwise(g, oracle.gemm_nt(A, B, sfA, sfB), what=f"tail int {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(384, 768, 2048), (256, 1280, 4096)])
def test_dense_tail_split_gaussian(M, N, K):
    w = synth.dense(M, N, K, seed_base=888000 + M)
    g = run_dense(w.A, w.B, w.sfA, w.sfB)
    rep = assert_parity(g, oracle.gemm_nt(w.A, w.B, w.sfA, w.sfB), what=f"tail {M}x{N}x{K}")
    print(f"tail {M}x{N}x{K}:", rep)


@pytest.mark.parametrize("M,N,K", [(65, 2112, 1024), (300, 528, 640), (1, 32, 128), (17, 4096, 256),
                                   (64, 2112, 1664), (33, 7168, 2048)])
def test_dense_gaussian_shapes(M, N, K):
    w = synth.dense(M, N, K, seed_base=777000 + M)
    g = run_dense(w.A, w.B, w.sfA, w.sfB)
    rep = assert_parity(g, oracle.gemm_nt(w.A, w.B, w.sfA, w.sfB), what=f"{M}x{N}x{K}")
    print(f"{M}x{N}x{K}:", rep)


def test_dense_one_hot_identity_doubling_bitwise():
    rng = np.random.default_rng(5)
    M, N, K = 96, 384, 384
    w = synth.dense(M, N, K, seed_base=555000)
    # one-hot rows of A: C row = one fp8 product per column, exact in bf16
    A1 = np.zeros((M, K), dtype=np.uint8)
    ks = rng.integers(0, K, M)
    A1[np.arange(M), ks] = rng.choice(INT_CODES[1:], M)
    sfA = np.ldexp(1.0, rng.integers(-3, 4, (M, K // 128))).astype(np.float32)
    assert_bitwise(run_dense(A1, w.B, sfA, w.sfB), oracle.gemm_nt(A1, w.B, sfA, w.sfB), "one-hot")
    # identity B
    I = np.zeros((K, K), dtype=np.uint8)
    I[np.arange(K), np.arange(K)] = 0x38
    ones = np.ones((3, 3), dtype=np.float32)
    assert_bitwise(run_dense(w.A, I, w.sfA, ones), oracle.gemm_nt(w.A, I, w.sfA, ones), "identity")
    # doubling a scale row of A doubles that output row exactly
    g0 = run_dense(w.A, w.B, w.sfA, w.sfB)
    sf2 = w.sfA.copy()
    sf2[7] *= 2
    sf2[64] *= 0.5
    g1 = run_dense(w.A, w.B, sf2, w.sfB)
    f0, f1 = gu_bf16(g0), gu_bf16(g1)
    assert np.array_equal(f1[7], 2 * f0[7]) and np.array_equal(f1[64], 0.5 * f0[64])
    keep = [i for i in range(M) if i not in (7, 64)]
    assert np.array_equal(g1[keep], g0[keep])


def gu_bf16(b):
    from tests.parity import bf16_to_f64
    return bf16_to_f64(b)


def test_dense_deterministic():
    w = synth.workload("dec2112")
    a = run_dense(w.A, w.B, w.sfA, w.sfB, seed=3)
    b = run_dense(w.A, w.B, w.sfA, w.sfB, seed=4)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("kind", ["dec32768", "tail_split", "contiguous", "masked"])
def test_deterministic_across_calls(kind):
    """Same inputs, same bits: split-K with its last-arriver reduction (64x32768x512
    and the dense tail split), and both grouped layouts with their device-side tile
    schedules, each called twice into differently filled outputs."""
    if kind in ("dec32768", "tail_split"):
        w = synth.workload("dec32768") if kind == "dec32768" else synth.dense(384, 768, 2048, 881000)
        a = run_dense(w.A, w.B, w.sfA, w.sfB, seed=5)
        b = run_dense(w.A, w.B, w.sfA, w.sfB, seed=6)
        assert np.array_equal(a, b)
    elif kind == "contiguous":
        counts = np.array([300, 0, 17, 129, 256, 1], dtype=np.int32)
        w = synth.contiguous(6, 512, 1024, 0, seed_base=882000, counts=counts)
        (a, _), (b, _) = (run_contiguous(w.A, w.B, w.sfA, w.sfB, w.m_indices, seed=s)
                          for s in (5, 6))
        pad = w.m_indices < 0
        assert np.array_equal(a[~pad], b[~pad])
    else:
        masked_m = np.array([200, 0, 77, 256, 31], dtype=np.int32)
        w = synth.masked(5, 256, 768, 1024, seed_base=883000, masked_m=masked_m)
        (a, _), (b, _) = (run_masked(w.A, w.B, w.sfA, w.sfB, w.masked_m, seed=s) for s in (5, 6))
        produced = np.arange(256)[None, :] < masked_m[:, None]
        assert np.array_equal(a[produced], b[produced])


@pytest.mark.parametrize("name", ["dec2112", "dec32768"])
def test_decode_workloads_full(name):
    w = synth.workload(name)
    g = run_dense(w.A, w.B, w.sfA, w.sfB)
    r = oracle.gemm_nt(w.A, w.B, w.sfA, w.sfB)
    rep = assert_parity(g, r, what=name)
    print(name, rep)
    model = assert_error_model(g, r, abs_product_sum(w.A, w.B, w.sfA, w.sfB), what=name)
    print(name, "error model:", model)


def test_decode_workloads_integer_exact_bitwise():
    for (M, N, K) in [(64, 2112, 7168), (64, 32768, 512)]:
        rng = np.random.default_rng(N)
        A, B, sfA, sfB = int_operands(rng, M, N, K)
        g = run_dense(A, B, sfA, sfB)
        assert_bitwise(g, oracle.gemm_nt(A, B, sfA, sfB), what=f"int {M}x{N}x{K}")


# ------------------------------------------------------------------ contiguous


def run_contiguous(A, B, sfA, sfB, m_indices, seed=2):
    M_total, K = A.shape
    G, N, _ = B.shape
    out = gu.Guarded((M_total, N), seed)
    gu.announce(f"contiguous M_total={M_total} N={N} K={K} G={G}")
    dg().m_grouped_fp8_gemm_nt_contiguous(gu.codes(A), gu.codes(B), out.out, gu.dev(sfA),
                                          gu.dev(sfB), gu.dev(m_indices.astype(np.int32)))
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside C"
    return out.result(), out.initial()


def check_contiguous_full(w, g, init, exact=False):
    r, produced = oracle.grouped_contiguous(w.A, w.B, w.sfA, w.sfB, w.m_indices)
    assert np.array_equal(g[~produced], init[~produced]), "pad rows touched"
    if exact:
        assert_bitwise(g[produced], r[produced], "contiguous int")
        return None
    return assert_parity(g[produced], r[produced], what="contiguous")


def test_contiguous_small_with_empty_experts():
    counts = np.array([5, 0, 128, 129, 0, 1, 300, 0], dtype=np.int32)
    w = synth.contiguous(8, 256, 384, 0, seed_base=888000, counts=counts)
    g, init = run_contiguous(w.A, w.B, w.sfA, w.sfB, w.m_indices)
    print("contiguous small:", check_contiguous_full(w, g, init))


def test_contiguous_unaligned_mixed_and_bad_ids_bitwise():
    rng = np.random.default_rng(17)
    G, N, K, M_total = 5, 144, 256, 300
    # experts interleaved inside 128-row groups, ids out of range, no alignment
    m_indices = rng.integers(-2, G + 2, size=M_total).astype(np.int32)
    m_indices[:40] = 3
    A, B, sfA, sfB = int_operands(rng, M_total, N, K, G=G)

    class W: pass
    w = W()
    w.A, w.B, w.sfA, w.sfB, w.m_indices = A, B, sfA, sfB, m_indices
    g, init = run_contiguous(A, B, sfA, sfB, m_indices)
    check_contiguous_full(w, g, init, exact=True)


def test_contiguous_nan_pad_rows_never_read():
    counts = np.array([3, 130, 0, 64], dtype=np.int32)
    w = synth.contiguous(4, 128, 256, 0, seed_base=889000, counts=counts,
                         pad_code=synth.FP8_NAN_CODE)
    assert np.any(w.A == synth.FP8_NAN_CODE)
    g, init = run_contiguous(w.A, w.B, w.sfA, w.sfB, w.m_indices)
    check_contiguous_full(w, g, init)


# ------------------------------------------------------------------ masked


def run_masked(A, B, sfA, sfB, masked_m, expected_m=None, seed=3):
    G, M_max, K = A.shape
    N = B.shape[1]
    out = gu.Guarded((G, M_max, N), seed)
    gu.announce(f"masked G={G} M_max={M_max} N={N} K={K}")
    dg().m_grouped_fp8_gemm_nt_masked(gu.codes(A), gu.codes(B), out.out, gu.dev(sfA),
                                      gu.dev(sfB), gu.dev(np.asarray(masked_m, np.int32)),
                                      expected_m)
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside C"
    return out.result(), out.initial()


def test_masked_partial_round_only():
    # 6 live tiles on a 16-workgroup grid (4 experts x 2 M-tiles x 2 N-tiles at full
    # height): the grid is mostly idle and one expert has a full 256-row pair of
    # tiles; integer-valued operands, so the result is exact
    rng = np.random.default_rng(41)
    G, M_max, N, K = 4, 256, 512, 1024
    masked_m = np.array([256, 0, 0, 10], dtype=np.int32)
    A, B, sfA, sfB = int_operands(rng, G * M_max, N, K, G=G)
    A, sfA = A.reshape(G, M_max, K), sfA.reshape(G, M_max, K // 128)
    g, init = run_masked(A, B, sfA, sfB, masked_m)
    r, produced = oracle.grouped_masked(A, B, sfA, sfB, masked_m)
    assert np.array_equal(g[~produced], init[~produced]), "masked rows touched"
    assert_bitwise(g[produced], r[produced], "masked partial round")


def test_masked_one_round_and_two_tiles():
    # 258 live tiles on the full 256-workgroup grid: one persistent round, then the
    # last expert's 2 tiles on two workgroups alone; that expert is checked in full,
    # the others at sampled positions; integer-valued operands
    rng = np.random.default_rng(43)
    G, M_max, N, K = 9, 2048, 512, 1024
    masked_m = np.array([2048] * 8 + [100], dtype=np.int32)
    A, B, sfA, sfB = int_operands(rng, G * M_max, N, K, G=G)
    A, sfA = A.reshape(G, M_max, K), sfA.reshape(G, M_max, K // 128)
    g, init = run_masked(A, B, sfA, sfB, masked_m)
    e = 8
    assert np.array_equal(g[e, 100:], init[e, 100:]), "masked rows touched"
    assert_bitwise(g[e, :100], oracle.gemm_nt(A[e, :100], B[e], sfA[e, :100], sfB[e]),
                   "masked, last expert")
    ei = rng.integers(0, 8, 3000)
    mi = rng.integers(0, M_max, 3000)
    ni = rng.integers(0, N, 3000)
    r = oracle.grouped_masked_at(A, B, sfA, sfB, masked_m, ei, mi, ni)
    assert_bitwise(g[ei, mi, ni], r, "masked whole tiles, sampled")


def test_masked_small_edges():
    masked_m = np.array([0, 200, 1, 129, 64, 65, 999, -4], dtype=np.int32)  # last two clamp
    w = synth.masked(8, 200, 256, 384, seed_base=990000, masked_m=masked_m,
                     pad_code=synth.FP8_NAN_CODE)
    g, init = run_masked(w.A, w.B, w.sfA, w.sfB, w.masked_m)
    r, produced = oracle.grouped_masked(w.A, w.B, w.sfA, w.sfB, w.masked_m)
    assert np.array_equal(g[~produced], init[~produced]), "masked rows touched"
    print("masked small:", assert_parity(g[produced], r[produced], what="masked small"))


def test_masked_integer_exact_bitwise():
    rng = np.random.default_rng(31)
    G, M_max, N, K = 4, 96, 2112, 512
    A, B, sfA, sfB = int_operands(rng, G * M_max, N, K, G=G)
    A = A.reshape(G, M_max, K)
    sfA = sfA.reshape(G, M_max, K // 128)
    masked_m = np.array([96, 33, 0, 64], dtype=np.int32)
    for em in (None, 16, 96):
        g, init = run_masked(A, B, sfA, sfB, masked_m, expected_m=em)
        r, produced = oracle.grouped_masked(A, B, sfA, sfB, masked_m)
        assert np.array_equal(g[~produced], init[~produced])
        assert_bitwise(g[produced], r[produced], "masked int")


def test_masked_32_row_boundaries_bitwise():
    # valid-row counts on both sides of every 32-row boundary of a 128-row tile: the
    # wave whose 64-row half holds 1..32 rows skips its second 32-row A tile
    rng = np.random.default_rng(57)
    masked_m = np.array([1, 31, 32, 33, 63, 64, 65, 95, 96, 97, 127, 128, 129, 160, 192, 200],
                        dtype=np.int32)
    G, M_max, N, K = masked_m.size, 256, 384, 512
    A, B, sfA, sfB = int_operands(rng, G * M_max, N, K, G=G)
    A, sfA = A.reshape(G, M_max, K), sfA.reshape(G, M_max, K // 128)
    for e in range(G):
        A[e, masked_m[e]:] = synth.FP8_NAN_CODE  # never read into an output
    g, init = run_masked(A, B, sfA, sfB, masked_m)
    r, produced = oracle.grouped_masked(A, B, sfA, sfB, masked_m)
    assert np.array_equal(g[~produced], init[~produced]), "masked rows touched"
    assert_bitwise(g[produced], r[produced], "masked 32-row boundaries")


def test_contiguous_32_row_boundaries_bitwise():
    # segment lengths ending on both sides of 32-row boundaries (pad rows fill each
    # segment to a multiple of 128)
    rng = np.random.default_rng(58)
    counts = np.array([1, 31, 32, 33, 64, 65, 96, 97, 127, 160], dtype=np.int32)
    G, N, K = counts.size, 272, 384
    m_indices = synth.contiguous_layout(counts)
    A, B, sfA, sfB = int_operands(rng, m_indices.size, N, K, G=G)
    A[m_indices < 0] = synth.FP8_NAN_CODE

    class W: pass
    w = W()
    w.A, w.B, w.sfA, w.sfB, w.m_indices = A, B, sfA, sfB, m_indices
    g, init = run_contiguous(A, B, sfA, sfB, m_indices)
    check_contiguous_full(w, g, init, exact=True)


def test_masked_many_experts_bitwise():
    # more than 64 experts: the device-side tile schedule scans the counts in
    # several 64-wide chunks; empty experts sit at chunk edges
    rng = np.random.default_rng(41)
    G, M_max, N, K = 70, 130, 272, 256
    A, B, sfA, sfB = int_operands(rng, G * M_max, N, K, G=G)
    A, sfA = A.reshape(G, M_max, K), sfA.reshape(G, M_max, K // 128)
    masked_m = rng.integers(0, M_max + 1, size=G).astype(np.int32)
    masked_m[[0, 63, 64, 69]] = [0, 0, 130, 0]
    g, init = run_masked(A, B, sfA, sfB, masked_m)
    r, produced = oracle.grouped_masked(A, B, sfA, sfB, masked_m)
    assert np.array_equal(g[~produced], init[~produced])
    assert_bitwise(g[produced], r[produced], "masked G=70")


def test_masked_all_empty_untouched():
    rng = np.random.default_rng(43)
    G, M_max, N, K = 5, 64, 144, 256
    A, B, sfA, sfB = int_operands(rng, G * M_max, N, K, G=G)
    A, sfA = A.reshape(G, M_max, K), sfA.reshape(G, M_max, K // 128)
    g, init = run_masked(A, B, sfA, sfB, np.array([0, -3, 0, 0, 0], dtype=np.int32))
    assert np.array_equal(g, init), "an all-empty call wrote output"


# ------------------------------------------------------------------ longest K


@pytest.mark.parametrize("M,K,cfg", [
    (130, 1 << 22, "pipe256x128"),  # the pipelined kernels' longest K (32-bit row offsets)
    (130, 1 << 22, "pipe128x256"),
    (64, 1 << 22, None),            # M <= 64: the split-K decode kernel
    (130, (1 << 22) + 128, None),   # one K-block past it: the generic tile kernel
])
def test_longest_k_sparse_blocks_bitwise(M, K, cfg, force_config):
    """Integer operands in five K-blocks (both ends and the middle), zeros elsewhere:
    every operand and scale address up to the last byte of the longest rows is read.
    Zero blocks add exact zeros, so the oracle runs on the five blocks alone."""
    if cfg:
        force_config(cfg)
    N, KB = 48, K // 128
    blocks = [0, 1, KB // 2, KB - 2, KB - 1]
    rng = np.random.default_rng(M + KB)
    a, b, sa, sb = int_operands(rng, M, N, 128 * len(blocks))
    A = np.zeros((M, K), np.uint8)
    B = np.zeros((N, K), np.uint8)
    sfA = np.ones((M, KB), np.float32)
    sfB = np.ones(((N + 127) // 128, KB), np.float32)
    for i, kb in enumerate(blocks):
        A[:, kb * 128:(kb + 1) * 128] = a[:, i * 128:(i + 1) * 128]
        B[:, kb * 128:(kb + 1) * 128] = b[:, i * 128:(i + 1) * 128]
        sfA[:, kb] = sa[:, i]
        sfB[:, kb] = sb[:, i]
    g = run_dense(A, B, sfA, sfB)
    assert_bitwise(g, oracle.gemm_nt(a, b, sa, sb), what=f"{cfg} {M}x{N}x{K}")


# ------------------------------------------------------------------ every configuration


@pytest.fixture
def force_config(monkeypatch):
    def set_cfg(name):
        monkeypatch.setenv("DG_FORCE_CONFIG", name)
    yield set_cfg


def all_configs():
    import fp8_block_scaled_dg_amd as m
    return m.config_names()


@pytest.mark.parametrize("cfg", all_configs())
def test_every_config_dense_integer_exact(cfg, force_config):
    force_config(cfg)
    shapes = [(64, 2112, 1024), (37, 272, 384), (1, 16, 128), (64, 2112, 1664), (50, 1040, 7168),
              # K runs of 3 and 2 blocks (64x8192x640: 128 column tiles, 2 splits) and of
              # 3 (48x16384x384: one split): the rolling kernel's loop and tail both run
              (64, 8192, 640), (48, 16384, 384)]
    if not cfg.startswith("skinny"):
        shapes += [(300, 400, 512), (129, 144, 256)]
    for (M, N, K) in shapes:
        rng = np.random.default_rng(M + N + K)
        A, B, sfA, sfB = int_operands(rng, M, N, K)
        g = run_dense(A, B, sfA, sfB)
        assert_bitwise(g, oracle.gemm_nt(A, B, sfA, sfB), what=f"{cfg} {M}x{N}x{K}")


@pytest.mark.parametrize("cfg", [c for c in all_configs() if not c.startswith("skinny")])
def test_every_config_grouped_integer_exact(cfg, force_config):
    force_config(cfg)
    rng = np.random.default_rng(3)
    G, N, K = 3, 272, 384
    counts = np.array([70, 0, 200], dtype=np.int32)
    m_indices = synth.contiguous_layout(counts)
    A, B, sfA, sfB = int_operands(rng, m_indices.size, N, K, G=G)

    class W: pass
    w = W()
    w.A, w.B, w.sfA, w.sfB, w.m_indices = A, B, sfA, sfB, m_indices
    g, init = run_contiguous(A, B, sfA, sfB, m_indices)
    check_contiguous_full(w, g, init, exact=True)
    M_max = 150
    Am, _, sfAm, _ = int_operands(rng, G * M_max, N, K, G=G)
    Am, sfAm = Am.reshape(G, M_max, K), sfAm.reshape(G, M_max, K // 128)
    masked_m = np.array([150, 0, 77], dtype=np.int32)
    g, init = run_masked(Am, B, sfAm, sfB, masked_m)
    r, produced = oracle.grouped_masked(Am, B, sfAm, sfB, masked_m)
    assert np.array_equal(g[~produced], init[~produced])
    assert_bitwise(g[produced], r[produced], f"{cfg} masked")
