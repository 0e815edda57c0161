"""CPU checks of the C ABI: libdg.so loads, exports every function include/dg.h
declares, and rejects bad arguments on the host before any HIP call (so these run
without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dg.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dg_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def dg():
    import fp8_block_scaled_dg_amd as m
    return m


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("dg_fp8_gemm_nt", "dg_m_grouped_fp8_gemm_nt_contiguous",
              "dg_m_grouped_fp8_gemm_nt_masked", "dg_status_string", "dg_last_error_detail"):
        assert n in names


def test_library_exports_every_declared_symbol(dg):
    out = subprocess.run(["nm", "-D", "--defined-only", dg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(\S+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    for n in declared_functions():
        assert hasattr(dg.lib, n)


def test_library_is_gfx950_code_object(dg):
    # the fat binary carries a gfx950 code object
    data = open(dg.LIB_PATH, "rb").read()
    assert b"gfx950" in data


FAKE = 0x10000  # a 16-byte-aligned non-NULL address; validation fails before any use


def call_dense(dg, A=FAKE, B=FAKE, C=FAKE, sA=FAKE, sB=FAKE, M=64, N=128, K=256):
    return dg.lib.dg_fp8_gemm_nt(A, B, C, sA, sB, M, N, K, None)


def status(dg, code):
    return dg.lib.dg_status_string(code).decode()


def test_dense_rejects_bad_arguments(dg):
    assert status(dg, call_dense(dg, A=None)) == "DG_ERR_NULL_POINTER"
    assert status(dg, call_dense(dg, sB=None)) == "DG_ERR_NULL_POINTER"
    assert status(dg, call_dense(dg, K=200)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, call_dense(dg, N=120)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, call_dense(dg, M=-1)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, call_dense(dg, K=0)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, call_dense(dg, A=FAKE + 8)) == "DG_ERR_MISALIGNED"
    assert status(dg, call_dense(dg, C=FAKE + 2)) == "DG_ERR_MISALIGNED"
    assert status(dg, call_dense(dg, sA=FAKE + 2)) == "DG_ERR_MISALIGNED"
    call_dense(dg, K=200)
    assert "128" in dg.lib.dg_last_error_detail().decode()


def test_zero_sized_work_is_a_noop(dg):
    # nothing to produce: DG_OK without touching any pointer or the GPU
    assert status(dg, call_dense(dg, A=None, B=None, C=None, sA=None, sB=None, M=0)) == "DG_OK"
    assert status(dg, call_dense(dg, A=None, B=None, C=None, sA=None, sB=None, N=0)) == "DG_OK"
    assert status(dg, dg.lib.dg_m_grouped_fp8_gemm_nt_contiguous(
        None, None, None, None, None, None, 0, 128, 256, 4, None)) == "DG_OK"
    assert status(dg, dg.lib.dg_m_grouped_fp8_gemm_nt_masked(
        None, None, None, None, None, None, 4, 0, 128, 256, 0, None)) == "DG_OK"


def test_grouped_reject_bad_arguments(dg):
    c = dg.lib.dg_m_grouped_fp8_gemm_nt_contiguous
    assert status(dg, c(FAKE, FAKE, FAKE, FAKE, FAKE, None, 128, 128, 256, 4, None)) == \
        "DG_ERR_NULL_POINTER"
    assert status(dg, c(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, 128, 256, 0, None)) == \
        "DG_ERR_BAD_SHAPE"
    assert status(dg, c(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE + 2, 128, 128, 256, 4, None)) == \
        "DG_ERR_MISALIGNED"
    m = dg.lib.dg_m_grouped_fp8_gemm_nt_masked
    assert status(dg, m(FAKE, FAKE, FAKE, FAKE, FAKE, None, 4, 64, 128, 256, 0, None)) == \
        "DG_ERR_NULL_POINTER"
    assert status(dg, m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 64, 128, 256, 0, None)) == \
        "DG_ERR_BAD_SHAPE"
    assert status(dg, m(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 4, 64, 128, 100, 0, None)) == \
        "DG_ERR_BAD_SHAPE"


def test_status_strings(dg):
    for code, name in enumerate(["DG_OK", "DG_ERR_NULL_POINTER", "DG_ERR_BAD_SHAPE",
                                 "DG_ERR_UNSUPPORTED_SHAPE", "DG_ERR_MISALIGNED",
                                 "DG_ERR_NO_DEVICE", "DG_ERR_LAUNCH", "DG_ERR_CAPTURE"]):
        assert status(dg, code) == name


def test_capture_status_is_declared():
    # a call that would allocate during a stream capture reports this status
    text = open(HEADER).read()
    assert re.search(r"DG_ERR_CAPTURE\s*=\s*7", text)


def test_build_id_matches_the_sources(dg):
    # the binding refuses a stale libdg.so; the id compiled in is the sources' hash
    from fp8_block_scaled_dg_amd import build
    assert dg.lib.dg_build_id().decode() == build.source_hash() == dg.BUILD_ID


def test_config_table_is_shape_keyed(dg):
    small = dg.describe_config(0, 64, 2112, 7168)
    big = dg.describe_config(0, 4096, 7168, 18432)
    assert small and big
    assert dg.describe_config(2, 256, 7168, 2048, 32, 120)
    with pytest.raises(dg.DGError):
        dg.describe_config(7, 1, 16, 128)


def test_binding_rejects_cpu_tensors(dg):
    import torch
    a = torch.zeros(64, 128, dtype=torch.float8_e4m3fn)
    b = torch.zeros(128, 128, dtype=torch.float8_e4m3fn)
    c = torch.zeros(64, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        dg.fp8_gemm_nt(a, b, c, torch.ones(64, 1), torch.ones(1, 1))
    with pytest.raises(TypeError):
        dg.fp8_gemm_nt(a.float(), b, c, torch.ones(64, 1), torch.ones(1, 1))


def test_quantizer_rejects_bad_arguments(dg):
    q = dg.lib.dg_quantize_fp8_1x128
    F32, BF16 = dg.DTYPE_F32, dg.DTYPE_BF16
    assert status(dg, q(None, F32, FAKE, FAKE, 4, 256, None)) == "DG_ERR_NULL_POINTER"
    assert status(dg, q(FAKE, BF16, FAKE, None, 4, 256, None)) == "DG_ERR_NULL_POINTER"
    assert status(dg, q(FAKE, F32, FAKE, FAKE, 4, 200, None)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, q(FAKE, F32, FAKE, FAKE, -1, 256, None)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, q(FAKE, 7, FAKE, FAKE, 4, 256, None)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, q(FAKE + 4, F32, FAKE, FAKE, 4, 256, None)) == "DG_ERR_MISALIGNED"
    assert status(dg, q(FAKE, F32, FAKE + 8, FAKE, 4, 256, None)) == "DG_ERR_MISALIGNED"
    assert status(dg, q(FAKE, F32, FAKE, FAKE + 2, 4, 256, None)) == "DG_ERR_MISALIGNED"
    assert status(dg, q(FAKE, F32, FAKE, FAKE, 1 << 36, 1 << 10, None)) == \
        "DG_ERR_UNSUPPORTED_SHAPE"
    # nothing to produce
    assert status(dg, q(None, F32, None, None, 0, 256, None)) == "DG_OK"
    assert status(dg, q(None, BF16, None, None, 4, 0, None)) == "DG_OK"


def test_quantizer_binding_checks_dtype_and_device(dg):
    import torch
    with pytest.raises(TypeError):
        dg.quantize_fp8_1x128(torch.zeros(2, 128, dtype=torch.float16, device="cpu"))
    with pytest.raises(ValueError):
        dg.quantize_fp8_1x128(torch.zeros(2, 128, dtype=torch.float32, device="cpu"))


def test_swiglu_calls_reject_bad_arguments(dg):
    c = dg.lib.dg_m_grouped_fp8_gemm_nt_contiguous_swiglu
    m = dg.lib.dg_m_grouped_fp8_gemm_nt_masked_swiglu
    F = FAKE
    assert status(dg, c(F, F, F, F, F, F, F, 128, 200, 256, 4, None)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, c(F, F, F, F, F, F, F, 128, 256, 200, 4, None)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, c(F, F, None, F, F, F, F, 128, 256, 256, 4, None)) == "DG_ERR_NULL_POINTER"
    assert status(dg, c(F, F, F + 4, F, F, F, F, 128, 256, 256, 4, None)) == "DG_ERR_MISALIGNED"
    assert status(dg, c(F, F, F, F, F, F, F, 128, 1 << 20, 1 << 12, 4, None)) == \
        "DG_ERR_UNSUPPORTED_SHAPE"
    assert status(dg, m(F, F, F, F, F, F, None, 4, 64, 256, 256, None)) == "DG_ERR_NULL_POINTER"
    assert status(dg, m(F, F, F, F, F, F, F, 0, 64, 256, 256, None)) == "DG_ERR_BAD_SHAPE"
    assert status(dg, c(None, None, None, None, None, None, None, 0, 256, 256, 4, None)) == "DG_OK"
