"""GPU: the allocation-free dense entry point, dg_fp8_gemm_nt_noalloc, called through
the C ABI, must give the same output as dg_fp8_gemm_nt, bit for bit: on two calls
in a row with the second smaller (the scratch array keeps the first call's bytes),
on the split-K decode kernel, the dense tail split and a skinny shape, and captured
into a HIP graph on a stream where nothing has run before (no allocation happens
under capture), replayed several times with eager work between the replays."""
import ctypes

import numpy as np
import pytest
import torch

from tests import gpu_util as gu
from tests.test_gpu_parity import int_operands

pytestmark = pytest.mark.gpu


def lib():
    import fp8_block_scaled_dg_amd as m
    return m.lib


def operands(M, N, K, seed):
    rng = np.random.default_rng(seed)
    A, B, sfA, sfB = int_operands(rng, M, N, K)
    # N(0,1)-like magnitudes are not needed: integer codes with power-of-two scales
    # make the two calls' equality a bitwise statement either way
    return gu.codes(A), gu.codes(B), gu.dev(sfA), gu.dev(sfB)


def call(fn, a, b, c, sa, sb, stream=None):
    M, K = a.shape
    N = b.shape[0]
    st = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    return fn(a.data_ptr(), b.data_ptr(), c.data_ptr(), sa.data_ptr(), sb.data_ptr(), M, N, K, st)


def both(M, N, K, seed):
    a, b, sa, sb = operands(M, N, K, seed)
    ref = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    got = torch.full((M, N), -3.0, dtype=torch.bfloat16, device="cuda")
    gu.announce(f"noalloc dense {M}x{N}x{K}")
    assert call(lib().dg_fp8_gemm_nt, a, b, ref, sa, sb) == 0
    assert call(lib().dg_fp8_gemm_nt_noalloc, a, b, got, sa, sb) == 0
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("first,second", [
    ((64, 2112, 7168), (64, 2112, 1024)),   # split-K decode kernel, then the skinny kernel
    ((384, 768, 2048), (256, 512, 1024)),   # compute-bound kernel with its tail split
    ((64, 32768, 512), (1, 16, 128)),
])
def test_noalloc_equals_allocating_call(first, second):
    for i, (M, N, K) in enumerate((first, second)):
        ref, got = both(M, N, K, seed=M + N + K + i)
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"{M}x{N}x{K}"


def test_noalloc_captured_on_a_fresh_stream():
    M, N, K = 64, 2112, 7168
    a, b, sa, sb = operands(M, N, K, 11)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    assert call(lib().dg_fp8_gemm_nt, a, b, ref, sa, sb) == 0
    torch.cuda.synchronize()
    got = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    gu.announce("noalloc under graph capture")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        rc = call(lib().dg_fp8_gemm_nt_noalloc, a, b, got, sa, sb, s.cuda_stream)
    assert rc == 0, lib().dg_last_error_detail()
    torch.cuda.synchronize()
    for rep in range(4):
        got.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(got.view(torch.int16), ref.view(torch.int16)), f"replay {rep}"
        # eager allocation-free calls between the replays, on another shape
        ref2, got2 = both(64, 4096, 512, seed=rep)
        assert torch.equal(got2.view(torch.int16), ref2.view(torch.int16))


def test_noalloc_rejects_bad_arguments_like_the_allocating_call():
    f = lib().dg_fp8_gemm_nt_noalloc
    f.restype = ctypes.c_int
    assert f(None, 0x10000, 0x10000, 0x10000, 0x10000, 64, 128, 256, None) == 1
    assert f(0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 64, 128, 200, None) == 2
