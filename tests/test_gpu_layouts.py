"""GPU parity of the NN / TN / TT dense GEMM calls (dg_fp8_gemm_nn / _tn / _tt): the
oracle's layout GEMM (strided indexing of the stored operands) must match bit for bit
on integer-valued inputs and within the tolerance on N(0,1) inputs; and each call
must equal dg_fp8_gemm_nt on transposed copies of its operands bit for bit, up to the
full prefill shape.

Two paths serve these calls. Shapes of the compute-bound kernel (M > 64) and of the
M <= 64 stream and rolling kernels read the [K][M] / [K][N] operands in place (k-row
tiles, transposing LDS reads): covered on both compute-bound tile shapes, two stream
and two rolling configurations, M and N tails, the dense tail split, split K, long K,
and by capture into a HIP graph on a fresh stream, which succeeds only because nothing
is allocated. A stored [K][M] with M % 16 != 0 goes through a transposed copy: odd M
covers that path."""
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


NATIVE = [(128, 256, 512), (144, 272, 384), (256, 1040, 1152), (384, 768, 2048),
          (208, 4096, 256), (320, 400, 8192)]


@pytest.mark.parametrize("cfg", ["pipe256x128", "pipe128x256"])
@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_native_layouts_every_tile_shape_bitwise(cfg, layout, monkeypatch):
    """In-place reads of MN-contiguous operands on both tile shapes: N tails of 16
    columns, M tails, the dense tail split (384x768x2048) and a long K."""
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    for (M, N, K) in NATIVE:
        rng = np.random.default_rng(M + 3 * N + 7 * K + ord(layout[0]) + 5 * ord(layout[1]))
        A_mk, B_nk, sfA, sfB = int_operands(rng, M, N, K)
        A, B = stored(A_mk, B_nk, layout)
        g = run(layout, A, B, sfA, sfB, M, N)
        assert_bitwise(g, oracle.gemm(A, B, sfA, sfB, layout), what=f"{cfg} {layout} {M}x{N}x{K}")
        assert np.array_equal(g, run("nt", A_mk, B_nk, sfA, sfB, M, N))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_native_layout_gaussian(layout):
    M, N, K = 208, 528, 1536
    w = synth.dense(M, N, K, 779000)
    A, B = stored(w.A, w.B, layout)
    g = run(layout, A, B, w.sfA, w.sfB, M, N)
    print(layout, assert_parity(g, oracle.gemm(A, B, w.sfA, w.sfB, layout), what=layout))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_native_layout_allocates_nothing(layout):
    """256x1024x512 (whole rounds of tiles, no split): captured into a HIP graph on a
    stream where nothing ran before. The copy path would need a workspace and fail
    with DG_ERR_CAPTURE; the in-place path records only its kernel."""
    import fp8_block_scaled_dg_amd as dg
    M, N, K = 256, 1024, 512
    rng = np.random.default_rng(11 + ord(layout[0]) + ord(layout[1]))
    A_mk, B_nk, sfA, sfB = int_operands(rng, M, N, K)
    A, B = stored(A_mk, B_nk, layout)
    a, b, sa, sb = gu.codes(A), gu.codes(B), gu.dev(sfA), gu.dev(sfB)
    c = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    gu.announce(f"native {layout} under capture")
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        getattr(dg, "fp8_gemm_" + layout)(a, b, c, sa, sb)
    for rep in range(3):
        c.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = c.view(torch.int16).cpu().numpy().view(np.uint16)
        assert_bitwise(got, oracle.gemm(A, B, sfA, sfB, layout), what=f"{layout} replay {rep}")


STREAM_MN = [(64, 2112, 7168), (64, 2112, 2048), (16, 272, 2560), (48, 80, 1280),
             (37, 96, 1536), (64, 32768, 512), (1, 16, 128), (32, 1072, 4096),
             (64, 2560, 2048)]


@pytest.mark.parametrize("cfg", ["stream_w4_tn1_d10", "stream_w4_tn1_d4"])
@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_stream_layouts_bitwise(cfg, layout, monkeypatch):
    """M <= 64 on the stream kernel: B stored [K][N] staged through the LDS ring, A
    stored [K][M] (M % 16 == 0) by DMA, both read transposed; the decode shape with its
    6-way split K, split K on short K, column tails of 16, 32 and 48, M = 1, 16, 37, 48
    (37: A stored [K][M] takes the copy path), one K-block; column tiles dealt to the
    XCDs in groups of 4 (2112 and 32768 columns), 2 (1072) and 1 (2560, 272). A
    configuration whose K run does not fit a shape falls back to the default choice
    (64x2112x7168 on the 4-block one)."""
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    for (M, N, K) in STREAM_MN:
        rng = np.random.default_rng(M + 5 * N + 3 * K + ord(layout[0]) + 7 * ord(layout[1]))
        A_mk, B_nk, sfA, sfB = int_operands(rng, M, N, K)
        A, B = stored(A_mk, B_nk, layout)
        g = run(layout, A, B, sfA, sfB, M, N)
        assert_bitwise(g, oracle.gemm(A, B, sfA, sfB, layout), what=f"{cfg} {layout} {M}x{N}x{K}")
        assert np.array_equal(g, run("nt", A_mk, B_nk, sfA, sfB, M, N))


@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_decode_layout_gaussian(layout):
    M, N, K = 64, 2112, 7168
    w = synth.dense(M, N, K, 780000)
    A, B = stored(w.A, w.B, layout)
    g = run(layout, A, B, w.sfA, w.sfB, M, N)
    print(layout, assert_parity(g, oracle.gemm(A, B, w.sfA, w.sfB, layout), what=layout))
    assert np.array_equal(g, run("nt", w.A, w.B, w.sfA, w.sfB, M, N))


SKINNY_MN = [(64, 32768, 512), (64, 2112, 1024), (16, 272, 384), (48, 80, 1280),
             (37, 96, 640), (1, 16, 128), (32, 1072, 896), (64, 2560, 256),
             (64, 8192, 640)]  # K runs of 3 and 2 blocks


@pytest.mark.parametrize("cfg", ["skinny_w4_tn1_d2", "skinny_w4_tn1_d8"])
@pytest.mark.parametrize("layout", ["nn", "tn", "tt"])
def test_rolling_layouts_bitwise(cfg, layout, monkeypatch):
    """M <= 64 on the rolling kernel: A stored [K][M] (M % 16 == 0) and B stored [K][N]
    staged into each block's LDS slot and read transposed; the 64x32768x512 decode
    shape, split K, column tails of 16 and 48, M = 1, 16, 32, 37, 48, 64 (37: A stored
    [K][M] takes the copy path), column tiles grouped 4, 2 and 1 per XCD."""
    monkeypatch.setenv("DG_FORCE_CONFIG", cfg)
    for (M, N, K) in SKINNY_MN:
        rng = np.random.default_rng(M + 7 * N + 5 * K + 3 * ord(layout[0]) + ord(layout[1]))
        A_mk, B_nk, sfA, sfB = int_operands(rng, M, N, K)
        A, B = stored(A_mk, B_nk, layout)
        g = run(layout, A, B, sfA, sfB, M, N)
        assert_bitwise(g, oracle.gemm(A, B, sfA, sfB, layout), what=f"{cfg} {layout} {M}x{N}x{K}")
        assert np.array_equal(g, run("nt", A_mk, B_nk, sfA, sfB, M, N))


def test_print_configs_names_the_layout_route(tmp_path):
    """DG_PRINT_CONFIGS=1 (read once per process, so in a child process): an NN call on
    the decode kernel reports "in place", a TN call with M % 16 != 0 "transposed copy"."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    script = tmp_path / "calls.py"
    script.write_text(
        "import sys\n"
        f"sys.path.insert(0, {root!r})\n"
        "import numpy as np, torch\n"
        "from tests import gpu_util as gu\n"
        "from tests.test_gpu_parity import int_operands\n"
        "import fp8_block_scaled_dg_amd as dg\n"
        "rng = np.random.default_rng(5)\n"
        "for lay, (M, N, K) in (('nn', (64, 2112, 2048)), ('tn', (37, 96, 1536))):\n"
        "    A, B, sfA, sfB = int_operands(rng, M, N, K)\n"
        "    A = np.ascontiguousarray(A.T) if lay[0] == 't' else A\n"
        "    B = np.ascontiguousarray(B.T) if lay[1] == 'n' else B\n"
        "    c = torch.empty((M, N), dtype=torch.bfloat16, device='cuda')\n"
        "    getattr(dg, 'fp8_gemm_' + lay)(gu.codes(A), gu.codes(B), c, gu.dev(sfA), gu.dev(sfB))\n"
        "torch.cuda.synchronize()\n")
    env = dict(os.environ, DG_PRINT_CONFIGS="1")
    gu.announce("DG_PRINT_CONFIGS child process")
    r = subprocess.run([sys.executable, str(script)], env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [x for x in r.stderr.splitlines() if x.startswith("[dg] dense")]
    assert any("M=64 N=2112 K=2048" in x and "(NN, in place)" in x for x in lines), lines
    assert any("M=37 N=96 K=1536" in x and "(TN, transposed copy)" in x for x in lines), lines
