"""GPU: the calls captured into a HIP graph (torch.cuda.CUDAGraph) on a stream where the
same shapes already ran, replayed several times with eager work and synchronisations
in between; every replay must reproduce the eager result bit for bit. Covered: the
split-K decode kernel (its arrival counters must be back at zero after every launch),
also reading B stored [K][N] and A stored [K][M] in place, the compute-bound kernel's
split tail, and the masked grouped call. The library
allocates nothing for a shape it has run on the stream before, so nothing but the
kernels is recorded."""
import numpy as np
import pytest
import torch

from tests import gpu_util as gu
from tests.test_gpu_parity import int_operands

pytestmark = pytest.mark.gpu


def dg():
    import fp8_block_scaled_dg_amd as m
    return m


def _dense(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A, B, sfA, sfB = int_operands(rng, M, N, K)
    a, b, sa, sb = gu.codes(A), gu.codes(B), gu.dev(sfA), gu.dev(sfB)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    return (lambda: dg().fp8_gemm_nt(a, b, c, sa, sb)), c


def _layout(layout, M, N, K, seed):
    """A stored [K][M] for layout[0] == 't', B stored [K][N] for layout[1] == 'n'."""
    rng = np.random.default_rng(seed)
    A, B, sfA, sfB = int_operands(rng, M, N, K)
    A = np.ascontiguousarray(A.T) if layout[0] == "t" else A
    B = np.ascontiguousarray(B.T) if layout[1] == "n" else B
    a, b, sa, sb = gu.codes(A), gu.codes(B), gu.dev(sfA), gu.dev(sfB)
    c = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    call = getattr(dg(), "fp8_gemm_" + layout)
    return (lambda: call(a, b, c, sa, sb)), c


def _masked(seed):
    rng = np.random.default_rng(seed)
    G, M_max, N, K = 6, 200, 512, 1024
    A, B, sfA, sfB = int_operands(rng, G * M_max, N, K, G=G)
    a = gu.codes(A.reshape(G, M_max, K))
    b = gu.codes(B)
    sa = gu.dev(sfA.reshape(G, M_max, K // 128))
    sb = gu.dev(sfB)
    mm = gu.dev(np.array([200, 0, 17, 129, 64, 1], dtype=np.int32))
    c = torch.zeros((G, M_max, N), dtype=torch.bfloat16, device="cuda")
    return (lambda: dg().m_grouped_fp8_gemm_nt_masked(a, b, c, sa, sb, mm)), c


@pytest.mark.parametrize("case", ["decode_splitk", "dense_tail_split", "masked",
                                  "decode_nn_in_place", "decode_tn_in_place"])
def test_graph_replays_match_eager(case):
    if case == "decode_splitk":
        fn, c = _dense(64, 2112, 7168, 5)
    elif case == "decode_nn_in_place":
        fn, c = _layout("nn", 64, 2112, 7168, 8)
    elif case == "decode_tn_in_place":
        fn, c = _layout("tn", 48, 1040, 4096, 9)
    elif case == "dense_tail_split":
        fn, c = _dense(384, 768, 2048, 6)
    else:
        fn, c = _masked(7)
    gu.announce(f"graph {case}")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        fn()  # sizes the library's buffers for this stream
        fn()
    torch.cuda.synchronize()
    eager = c.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fn()
    torch.cuda.synchronize()
    for rep in range(4):
        c.zero_()  # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), eager.view(torch.int16)), f"{case}: replay {rep} differs"
        with torch.cuda.stream(s):
            fn()  # an eager call on the same stream between replays
        torch.cuda.synchronize()
        assert torch.equal(c.view(torch.int16), eager.view(torch.int16)), f"{case}: eager call after replay {rep} differs"


def test_capture_that_would_allocate_reports_capture_status():
    """On a stream where no split-K call has run, the library would have to allocate
    its workspace: under capture the call returns DG_ERR_CAPTURE and records nothing,
    and the same call then runs eagerly and, once warmed, captures fine."""
    fn, c = _dense(64, 2112, 7168, 8)
    gu.announce("graph capture before warm-up")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    err = None
    with torch.cuda.graph(g, stream=s):
        try:
            fn()
        except dg().DGError as e:
            err = e
    torch.cuda.synchronize()
    assert err is not None and err.status == 7, err
    assert "captur" in str(err)
    with torch.cuda.stream(s):
        fn()
    torch.cuda.synchronize()
    eager = c.clone()
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2, stream=s):
        fn()
    c.zero_()
    torch.cuda.synchronize()
    g2.replay()
    torch.cuda.synchronize()
    assert torch.equal(c.view(torch.int16), eager.view(torch.int16))


def test_replay_after_workspace_growth():
    """A graph captured on a small split-K shape keeps working after a larger shape has
    grown the stream's workspace: the outgrown buffer is retired, not freed."""
    small, c_small = _dense(64, 2112, 1024, 9)
    big, c_big = _dense(64, 2112, 7168, 10)
    gu.announce("graph replay after workspace growth")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        small()
    torch.cuda.synchronize()
    eager = c_small.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        small()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        big()  # grows the partials buffer of this stream
    torch.cuda.synchronize()
    eager_big = c_big.clone()
    for rep in range(3):
        c_small.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(c_small.view(torch.int16), eager.view(torch.int16)), f"replay {rep}"
        with torch.cuda.stream(s):
            big()
        torch.cuda.synchronize()
        assert torch.equal(c_big.view(torch.int16), eager_big.view(torch.int16))
