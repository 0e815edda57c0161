"""GPU parity of the NN / TN / TT dense GEMM calls (dg_fp8_gemm_nn / _tn / _tt): the
oracle's layout GEMM (strided indexing of the stored operands) must match bit for bit
on integer-valued inputs and within the tolerance on N(0,1) inputs; and each call
must equal dg_fp8_gemm_nt on transposed copies of its operands bit for bit, up to the
full prefill shape. Shapes cover odd M (the transposition's unaligned path), N tails,
M = 1, and M <= 64 (decode kernels) as well as the compute-bound kernel."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu
from tests.parity import assert_bitwise, assert_parity
from tests.test_gpu_parity import int_operands

pytestmark = pytest.mark.gpu


def stored(A_mk, B_nk, layout):
    A = np.ascontiguousarray(A_mk.T) if layout[0] == "t" else A_mk
    B = np.ascontiguousarray(B_nk.T) if layout[1] == "n" else B_nk
    return A, B


def run(layout, A, B, sfA, sfB, M, N, seed=2):
    import fp8_block_scaled_dg_amd as dg
    out = gu.Guarded((M, N), seed)
    gu.announce(f"dense {layout} M={M} N={N} K={sfA.shape[1] * 128}")
    getattr(dg, "fp8_gemm_" + layout)(gu.codes(A), gu.codes(B), out.out, gu.dev(sfA), gu.dev(sfB))
    torch.cuda.synchronize()
    assert out.guards_intact(), "write outside C"
    return out.result()


SHAPES = [(1, 16, 128), (37, 272, 384), (64, 2112, 1024), (130, 144, 256), (300, 400, 512),
          (517, 1040, 1152)]


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
@pytest.mark.parametrize("M,N,K", SHAPES)
def test_layout_integer_exact_bitwise(layout, M, N, K):
    rng = np.random.default_rng(M * 3 + N + K + ord(layout[0]) * 7 + ord(layout[1]))
    A_mk, B_nk, sfA, sfB = int_operands(rng, M, N, K)
    A, B = stored(A_mk, B_nk, layout)
    g = run(layout, A, B, sfA, sfB, M, N)
    assert_bitwise(g, oracle.gemm(A, B, sfA, sfB, layout), what=f"{layout} {M}x{N}x{K}")
    g_nt = run("nt", A_mk, B_nk, sfA, sfB, M, N)
    assert np.array_equal(g, g_nt)


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_layout_gaussian(layout):
    M, N, K = 200, 528, 1536
    w = synth.dense(M, N, K, 778000)
    A, B = stored(w.A, w.B, layout)
    g = run(layout, A, B, w.sfA, w.sfB, M, N)
    print(layout, assert_parity(g, oracle.gemm(A, B, w.sfA, w.sfB, layout), what=layout))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_prefill_shape_equals_nt(layout):
    # 4096x7168x18432: the transposed copies are 75.5 MB (A) and 132 MB (B)
    w = synth.workload("prefill")
    M, N, K = w.shape
    A, B = stored(w.A, w.B, layout)
    assert np.array_equal(run(layout, A, B, w.sfA, w.sfB, M, N),
                          run("nt", w.A, w.B, w.sfA, w.sfB, M, N))
