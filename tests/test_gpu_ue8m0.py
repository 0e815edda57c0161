"""GPU parity of the packed UE8M0 sfA layout (the *_ue8m0 calls).

The packed form re-encodes power-of-two scales, so a call with packed sfA must give
the same bf16 output, bit for bit, as the same call with the fp32 scales -- on every
compiled configuration, at K-block counts that do not fill the last word, and where
a workgroup's K range starts inside a word (split-K decode, dense tail split). With
integer-valued codes the output must also equal the oracle (fed the unpacked scales)
bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu
from tests.parity import assert_bitwise
from tests.test_gpu_parity import int_operands

pytestmark = pytest.mark.gpu


def dense_both(A, B, sfA, sfB, seed=1):
    import fp8_block_scaled_dg_amd as dg
    M, K = A.shape
    N = B.shape[0]
    outs = []
    for packed in (False, True):
        out = gu.Guarded((M, N), seed)
        a_sf = gu.dev(synth.pack_ue8m0(sfA)) if packed else gu.dev(sfA)
        gu.announce(f"dense {'ue8m0' if packed else 'fp32'} M={M} N={N} K={K}")
        dg.fp8_gemm_nt(gu.codes(A), gu.codes(B), out.out, a_sf, gu.dev(sfB))
        torch.cuda.synchronize()
        assert out.guards_intact(), "write outside C"
        outs.append(out.result())
    return outs


@pytest.fixture
def force_config(monkeypatch):
    def set_cfg(name):
        monkeypatch.setenv("DG_FORCE_CONFIG", name)
    yield set_cfg


def all_configs():
    import fp8_block_scaled_dg_amd as m
    return m.config_names()


@pytest.mark.parametrize("cfg", all_configs())
def test_every_config_dense_packed_equals_fp32(cfg, force_config):
    force_config(cfg)
    # K-blocks 3, 5, 13, 56 (words 1, 2, 4, 14); 64-row decode shapes and larger ones
    shapes = [(64, 2112, 1664), (37, 272, 384), (1, 16, 640), (50, 1040, 7168)]
    if not cfg.startswith("skinny") and not cfg.startswith("stream"):
        shapes += [(300, 400, 512), (129, 144, 640)]
    for (M, N, K) in shapes:
        rng = np.random.default_rng(M * 7 + N + K)
        A, B, sfA, sfB = int_operands(rng, M, N, K)
        g32, g8 = dense_both(A, B, sfA, sfB)
        assert np.array_equal(g32, g8), f"{cfg} {M}x{N}x{K}: packed sfA changed the output"
        r = oracle.gemm_nt(A, B, oracle.unpack_ue8m0(synth.pack_ue8m0(sfA), K // 128), sfB)
        assert_bitwise(g8, r, what=f"{cfg} {M}x{N}x{K} ue8m0")


@pytest.mark.parametrize("name", ["dec2112", "dec32768"])
def test_decode_workloads_packed_equals_fp32(name):
    # the default configuration: split-K runs start at K-blocks 0, 10, 20, ... (inside
    # words) for 64x2112x7168
    w = synth.workload(name)
    g32, g8 = dense_both(w.A, w.B, w.sfA, w.sfB)
    assert np.array_equal(g32, g8)


def test_dense_tail_split_packed_equals_fp32():
    # the compute-bound kernel's tail split: K parts start at part * KB / parts
    for (M, N, K) in [(384, 768, 2048), (300, 704, 3072), (256, 1280, 4224)]:
        rng = np.random.default_rng(M + N + K)
        A, B, sfA, sfB = int_operands(rng, M, N, K)
        g32, g8 = dense_both(A, B, sfA, sfB)
        assert np.array_equal(g32, g8), f"{M}x{N}x{K}"


def test_prefill_workload_packed_equals_fp32():
    w = synth.workload("prefill")
    g32, g8 = dense_both(w.A, w.B, w.sfA, w.sfB)
    assert np.array_equal(g32, g8)


def test_grouped_workloads_packed_equal_fp32():
    import fp8_block_scaled_dg_amd as dg
    w = synth.workload("moe_cont")
    M_total, N, K, G = w.shape
    res = []
    for packed in (False, True):
        out = gu.Guarded((M_total, N), 3)
        a_sf = gu.dev(synth.pack_ue8m0(w.sfA)) if packed else gu.dev(w.sfA)
        gu.announce(f"contiguous {'ue8m0' if packed else 'fp32'} workload")
        dg.m_grouped_fp8_gemm_nt_contiguous(gu.codes(w.A), gu.codes(w.B), out.out, a_sf,
                                            gu.dev(w.sfB), gu.dev(w.m_indices))
        torch.cuda.synchronize()
        assert out.guards_intact()
        res.append(out.result())
    assert np.array_equal(res[0], res[1])
    w = synth.workload("moe_mask", pad_code=synth.FP8_NAN_CODE)
    G, M_max, N, K = w.shape
    res = []
    for packed in (False, True):
        out = gu.Guarded((G, M_max, N), 4)
        a_sf = gu.dev(synth.pack_ue8m0(w.sfA)) if packed else gu.dev(w.sfA)
        gu.announce(f"masked {'ue8m0' if packed else 'fp32'} workload")
        dg.m_grouped_fp8_gemm_nt_masked(gu.codes(w.A), gu.codes(w.B), out.out, a_sf,
                                        gu.dev(w.sfB), gu.dev(w.masked_m))
        torch.cuda.synchronize()
        assert out.guards_intact()
        res.append(out.result())
    assert np.array_equal(res[0], res[1])


def test_grouped_small_packed_bitwise_vs_oracle():
    import fp8_block_scaled_dg_amd as dg
    rng = np.random.default_rng(23)
    G, N, K = 3, 272, 640  # 5 K-blocks: two words per row, the last one part-filled
    counts = np.array([70, 0, 200], dtype=np.int32)
    m_indices = synth.contiguous_layout(counts)
    A, B, sfA, sfB = int_operands(rng, m_indices.size, N, K, G=G)
    out = gu.Guarded((m_indices.size, N), 5)
    dg.m_grouped_fp8_gemm_nt_contiguous(gu.codes(A), gu.codes(B), out.out,
                                        gu.dev(synth.pack_ue8m0(sfA)), gu.dev(sfB), gu.dev(m_indices))
    torch.cuda.synchronize()
    g, init = out.result(), out.initial()
    r, produced = oracle.grouped_contiguous(A, B, oracle.unpack_ue8m0(synth.pack_ue8m0(sfA), K // 128),
                                            sfB, m_indices)
    assert np.array_equal(g[~produced], init[~produced])
    assert_bitwise(g[produced], r[produced], "contiguous ue8m0")
    M_max = 150
    Am, _, sfAm, _ = int_operands(rng, G * M_max, N, K, G=G)
    Am, sfAm = Am.reshape(G, M_max, K), sfAm.reshape(G, M_max, K // 128)
    masked_m = np.array([150, 0, 77], dtype=np.int32)
    out = gu.Guarded((G, M_max, N), 6)
    dg.m_grouped_fp8_gemm_nt_masked(gu.codes(Am), gu.codes(B), out.out,
                                    gu.dev(synth.pack_ue8m0(sfAm)), gu.dev(sfB), gu.dev(masked_m))
    torch.cuda.synchronize()
    g, init = out.result(), out.initial()
    r, produced = oracle.grouped_masked(Am, B, oracle.unpack_ue8m0(synth.pack_ue8m0(sfAm), K // 128),
                                        sfB, masked_m)
    assert np.array_equal(g[~produced], init[~produced])
    assert_bitwise(g[produced], r[produced], "masked ue8m0")
