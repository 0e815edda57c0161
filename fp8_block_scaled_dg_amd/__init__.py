"""Python binding of libdg.so, the MI355X (gfx950) FP8 block-scaled GEMM library.

Argument marshalling only: every call checks dtypes, devices, shapes and contiguity,
then passes raw device pointers and torch's current HIP stream to the C ABI declared
in ``include/dg.h``. All arithmetic runs in the library's HIP kernels; there is no
fallback path. If libdg.so is missing the import fails.

Calls (DeepGEMM project page, aiproducthub.cn, "quick start"; DeepGEMM launch
article, deepseek.csdn.net, section 4.2 "advanced tuning"):

* ``fp8_gemm_nt(a, b, c, a_sf, b_sf)`` and ``fp8_gemm_nn / _tn / _tt`` (other layouts)
* ``m_grouped_fp8_gemm_nt_contiguous(a, b, c, a_sf, b_sf, m_indices)``
* ``m_grouped_fp8_gemm_nt_masked(a, b, c, a_sf, b_sf, masked_m, expected_m=None)``
* ``quantize_fp8_1x128(x, codes=None, sf=None)``: activations -> (A codes, sfA)
* ``m_grouped_fp8_gemm_nt_{contiguous,masked}_swiglu(...)``: Linear1 with a fused
  SwiGLU + requantization epilogue -> (codes, sf) of h = silu(gate) * up

Operands: ``a``/``b`` are ``torch.float8_e4m3fn`` (``torch.uint8`` holding e4m3fn
codes is accepted too), ``a_sf``/``b_sf`` ``torch.float32``, ``c`` ``torch.bfloat16``
and the index tensors ``torch.int32``, all on the same GPU. An ``a_sf`` of dtype
``torch.int32`` and last dimension ceil(K/512) is the packed UE8M0 layout (one
exponent byte per K-block, four per word) and selects the ``*_ue8m0`` calls.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first: the library then binds to torch's HIP runtime

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdg.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python fp8_block_scaled_dg_amd/build.py` (hipcc, gfx950)")

_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32

lib = ctypes.CDLL(LIB_PATH)
lib.dg_build_id.restype = ctypes.c_char_p
lib.dg_build_id.argtypes = []
BUILD_ID = lib.dg_build_id().decode()


def _check_current() -> None:
    """Refuse a libdg.so built from other sources than the ones beside it."""
    from . import build as _build
    try:
        want = _build.source_hash()
    except OSError:  # sources not shipped: nothing to compare with
        return
    if want != BUILD_ID:
        raise ImportError(f"{LIB_PATH} was built from other sources (build id {BUILD_ID}, "
                          f"sources {want}); rebuild it: python fp8_block_scaled_dg_amd/build.py")


_check_current()
lib.dg_fp8_gemm_nt.restype = ctypes.c_int
lib.dg_fp8_gemm_nt.argtypes = [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _vp]
lib.dg_m_grouped_fp8_gemm_nt_contiguous.restype = ctypes.c_int
lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64,
                                                    _i64, _i32, _vp]
lib.dg_m_grouped_fp8_gemm_nt_masked.restype = ctypes.c_int
lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i64,
                                                _i64, _i64, _vp]
lib.dg_status_string.restype = ctypes.c_char_p
lib.dg_status_string.argtypes = [ctypes.c_int]
lib.dg_last_error_detail.restype = ctypes.c_char_p
lib.dg_last_error_detail.argtypes = []
lib.dg_describe_config.restype = ctypes.c_int
lib.dg_describe_config.argtypes = [_i32, _i64, _i64, _i64, _i32, _i64, ctypes.c_char_p, _i64]

lib.dg_fp8_gemm_nt_noalloc.restype = ctypes.c_int
lib.dg_fp8_gemm_nt_noalloc.argtypes = lib.dg_fp8_gemm_nt.argtypes
lib.dg_fp8_gemm_nt_ue8m0.restype = ctypes.c_int
lib.dg_fp8_gemm_nt_ue8m0.argtypes = lib.dg_fp8_gemm_nt.argtypes
lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0.restype = ctypes.c_int
lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0.argtypes = \
    lib.dg_m_grouped_fp8_gemm_nt_contiguous.argtypes
lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0.restype = ctypes.c_int
lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0.argtypes = lib.dg_m_grouped_fp8_gemm_nt_masked.argtypes
lib.dg_m_grouped_fp8_gemm_nt_contiguous_swiglu.restype = ctypes.c_int
lib.dg_m_grouped_fp8_gemm_nt_contiguous_swiglu.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                                          _i64, _i64, _i64, _i32, _vp]
lib.dg_m_grouped_fp8_gemm_nt_masked_swiglu.restype = ctypes.c_int
lib.dg_m_grouped_fp8_gemm_nt_masked_swiglu.argtypes = [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32,
                                                      _i64, _i64, _i64, _vp]
for _name in ("dg_fp8_gemm_nn", "dg_fp8_gemm_tn", "dg_fp8_gemm_tt"):
    getattr(lib, _name).restype = ctypes.c_int
    getattr(lib, _name).argtypes = lib.dg_fp8_gemm_nt.argtypes
lib.dg_quantize_fp8_1x128.restype = ctypes.c_int
lib.dg_quantize_fp8_1x128.argtypes = [_vp, _i32, _vp, _vp, _i64, _i64, _vp]

lib.dg_release_workspaces.restype = ctypes.c_int
lib.dg_release_workspaces.argtypes = []
lib.dg_num_configs.restype = _i32
lib.dg_num_configs.argtypes = []
lib.dg_config_name.restype = ctypes.c_char_p
lib.dg_config_name.argtypes = [_i32]

KIND_DENSE, KIND_CONTIGUOUS, KIND_MASKED = 0, 1, 2
DTYPE_F32, DTYPE_BF16 = 0, 1
BLOCK = 128


class DGError(RuntimeError):
    def __init__(self, status: int):
        self.status = status
        name = lib.dg_status_string(status).decode()
        detail = lib.dg_last_error_detail().decode()
        super().__init__(f"{name}: {detail}" if detail else name)


def check(status: int) -> None:
    if status != 0:
        raise DGError(status)


def _fp8(t: torch.Tensor, name: str) -> torch.Tensor:
    if t.dtype not in (torch.float8_e4m3fn, torch.uint8):
        raise TypeError(f"{name} must be torch.float8_e4m3fn (or uint8 codes), got {t.dtype}")
    return t


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple, device) -> None:
    # one combined test on the common path; the specific error only on failure
    if t.dtype != dtype or t.shape != shape or t.device != device or not t.is_contiguous():
        if t.dtype != dtype:
            raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        _dev(t, name, device)


def _dev(t: torch.Tensor, name: str, device) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_current_device = torch.cuda.current_device
_raw_stream = torch._C._cuda_getCurrentRawStream


def _run(dev, fn, *args) -> None:
    """fn(*args, stream): the library call on torch's current stream of `dev`, with
    `dev` the current device (the library keeps its workspace per device and stream).
    The device is switched only when it is not current already. Raises DGError on a
    nonzero status."""
    idx = dev.index
    if _current_device() == idx:
        status = fn(*args, _raw_stream(idx))
    else:
        with torch.cuda.device(idx):
            status = fn(*args, _raw_stream(idx))
    if status:
        raise DGError(status)


def _a_sf_layout(a_sf, lead: tuple, K: int, dev):
    """(packed?, expected shape) of a_sf: torch.float32 [..., K/128], or torch.int32
    [..., ceil(K/512)] holding packed UE8M0 bytes (one per K-block, 4 per word)."""
    if a_sf.dtype == torch.int32:
        shape = lead + ((K // BLOCK + 3) // 4,)
        _need(a_sf, "a_sf", torch.int32, shape, dev)
        return True
    _need(a_sf, "a_sf", torch.float32, lead + (K // BLOCK,), dev)
    return False


def fp8_gemm_nt(a, b, c, a_sf, b_sf) -> None:
    """c[M][N] (bf16) = block-scaled a[M][K] x b[N][K]^T; writes c in place. a_sf is
    fp32 [M, K/128], or int32 [M, ceil(K/512)] in the packed UE8M0 layout."""
    _fp8(a, "a"), _fp8(b, "b")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = a.shape
    N = b.shape[0]
    dev = a.device
    _dev(a, "a", dev)
    _need(b, "b", b.dtype, (N, K), dev)
    _need(c, "c", torch.bfloat16, (M, N), dev)
    packed = _a_sf_layout(a_sf, (M,), K, dev)
    _need(b_sf, "b_sf", torch.float32, ((N + BLOCK - 1) // BLOCK, K // BLOCK), dev)
    fn = lib.dg_fp8_gemm_nt_ue8m0 if packed else lib.dg_fp8_gemm_nt
    _run(dev, fn, a.data_ptr(), b.data_ptr(), c.data_ptr(), a_sf.data_ptr(), b_sf.data_ptr(),
         M, N, K)


def _fp8_gemm_layout(layout: str, a, b, c, a_sf, b_sf) -> None:
    _fp8(a, "a"), _fp8(b, "b")
    if a.dim() != 2 or b.dim() != 2:
        raise ValueError("a and b must be 2-D")
    M, K = (a.shape[1], a.shape[0]) if layout[0] == "t" else tuple(a.shape)
    N = b.shape[1] if layout[1] == "n" else b.shape[0]
    dev = a.device
    _dev(a, "a", dev)
    _need(b, "b", b.dtype, (K, N) if layout[1] == "n" else (N, K), dev)
    _need(c, "c", torch.bfloat16, (M, N), dev)
    _need(a_sf, "a_sf", torch.float32, (M, K // BLOCK), dev)
    _need(b_sf, "b_sf", torch.float32, ((N + BLOCK - 1) // BLOCK, K // BLOCK), dev)
    fn = getattr(lib, "dg_fp8_gemm_" + layout)
    _run(dev, fn, a.data_ptr(), b.data_ptr(), c.data_ptr(), a_sf.data_ptr(), b_sf.data_ptr(),
         M, N, K)


def fp8_gemm_nn(a, b, c, a_sf, b_sf) -> None:
    """c [M][N] = a [M][K] x b [K][N] (block-scaled; scales as for fp8_gemm_nt)."""
    _fp8_gemm_layout("nn", a, b, c, a_sf, b_sf)


def fp8_gemm_tn(a, b, c, a_sf, b_sf) -> None:
    """c [M][N] = a [K][M]^T x b [K][N]."""
    _fp8_gemm_layout("tn", a, b, c, a_sf, b_sf)


def fp8_gemm_tt(a, b, c, a_sf, b_sf) -> None:
    """c [M][N] = a [K][M]^T x b [N][K]^T."""
    _fp8_gemm_layout("tt", a, b, c, a_sf, b_sf)


def m_grouped_fp8_gemm_nt_contiguous(a, b, c, a_sf, b_sf, m_indices) -> None:
    """Contiguous MoE layout: row r of a uses expert m_indices[r]'s b (-1 = pad row,
    left untouched in c)."""
    _fp8(a, "a"), _fp8(b, "b")
    if a.dim() != 2 or b.dim() != 3:
        raise ValueError("a must be [M_total, K] and b [G, N, K]")
    M, K = a.shape
    G, N = b.shape[0], b.shape[1]
    dev = a.device
    _dev(a, "a", dev)
    _need(b, "b", b.dtype, (G, N, K), dev)
    _need(c, "c", torch.bfloat16, (M, N), dev)
    packed = _a_sf_layout(a_sf, (M,), K, dev)
    _need(b_sf, "b_sf", torch.float32, (G, (N + BLOCK - 1) // BLOCK, K // BLOCK), dev)
    _need(m_indices, "m_indices", torch.int32, (M,), dev)
    fn = (lib.dg_m_grouped_fp8_gemm_nt_contiguous_ue8m0 if packed
          else lib.dg_m_grouped_fp8_gemm_nt_contiguous)
    _run(dev, fn, a.data_ptr(), b.data_ptr(), c.data_ptr(), a_sf.data_ptr(), b_sf.data_ptr(),
         m_indices.data_ptr(), M, N, K, G)


def m_grouped_fp8_gemm_nt_masked(a, b, c, a_sf, b_sf, masked_m, expected_m=None) -> None:
    """Masked MoE layout: expert e computes its first masked_m[e] rows of a[e]; the
    other rows of c[e] are left untouched."""
    _fp8(a, "a"), _fp8(b, "b")
    if a.dim() != 3 or b.dim() != 3:
        raise ValueError("a must be [G, M_max, K] and b [G, N, K]")
    G, M_max, K = a.shape
    N = b.shape[1]
    dev = a.device
    _dev(a, "a", dev)
    _need(b, "b", b.dtype, (G, N, K), dev)
    _need(c, "c", torch.bfloat16, (G, M_max, N), dev)
    packed = _a_sf_layout(a_sf, (G, M_max), K, dev)
    _need(b_sf, "b_sf", torch.float32, (G, (N + BLOCK - 1) // BLOCK, K // BLOCK), dev)
    _need(masked_m, "masked_m", torch.int32, (G,), dev)
    em = int(expected_m) if expected_m is not None else 0
    fn = lib.dg_m_grouped_fp8_gemm_nt_masked_ue8m0 if packed else lib.dg_m_grouped_fp8_gemm_nt_masked
    _run(dev, fn, a.data_ptr(), b.data_ptr(), c.data_ptr(), a_sf.data_ptr(), b_sf.data_ptr(),
         masked_m.data_ptr(), G, M_max, N, K, em)


def _swiglu_outputs(lead: tuple, I: int, codes, sf, dev):
    if codes is None:
        codes = torch.empty(lead + (I,), dtype=torch.float8_e4m3fn, device=dev)
    if sf is None:
        sf = torch.empty(lead + (I // BLOCK,), dtype=torch.float32, device=dev)
    _fp8(codes, "codes")
    _need(codes, "codes", codes.dtype, lead + (I,), dev)
    _need(sf, "sf", torch.float32, lead + (I // BLOCK,), dev)
    return codes, sf


def m_grouped_fp8_gemm_nt_contiguous_swiglu(a, b, a_sf, b_sf, m_indices, codes=None, sf=None):
    """Contiguous MoE Linear1 with the fused SwiGLU + 1x128 requantization epilogue.
    b is [G, 2I, K] (gate rows, then up rows); returns (codes [M_total, I] e4m3fn,
    sf [M_total, I/128] fp32) of h = silu(gate) * up, written into the given tensors
    when passed. Pad rows are not written."""
    _fp8(a, "a"), _fp8(b, "b")
    if a.dim() != 2 or b.dim() != 3 or b.shape[1] % 2:
        raise ValueError("a must be [M_total, K] and b [G, 2I, K]")
    M, K = a.shape
    G, N2 = b.shape[0], b.shape[1]
    I = N2 // 2
    dev = a.device
    _dev(a, "a", dev)
    _need(b, "b", b.dtype, (G, N2, K), dev)
    _need(a_sf, "a_sf", torch.float32, (M, K // BLOCK), dev)
    _need(b_sf, "b_sf", torch.float32, (G, N2 // BLOCK, K // BLOCK), dev)
    _need(m_indices, "m_indices", torch.int32, (M,), dev)
    codes, sf = _swiglu_outputs((M,), I, codes, sf, dev)
    _run(dev, lib.dg_m_grouped_fp8_gemm_nt_contiguous_swiglu, a.data_ptr(), b.data_ptr(),
         codes.data_ptr(), sf.data_ptr(), a_sf.data_ptr(), b_sf.data_ptr(), m_indices.data_ptr(),
         M, I, K, G)
    return codes, sf


def m_grouped_fp8_gemm_nt_masked_swiglu(a, b, a_sf, b_sf, masked_m, codes=None, sf=None):
    """Masked MoE Linear1 with the fused SwiGLU + 1x128 requantization epilogue:
    returns (codes [G, M_max, I], sf [G, M_max, I/128]); rows >= masked_m[e] are not
    written."""
    _fp8(a, "a"), _fp8(b, "b")
    if a.dim() != 3 or b.dim() != 3 or b.shape[1] % 2:
        raise ValueError("a must be [G, M_max, K] and b [G, 2I, K]")
    G, M_max, K = a.shape
    N2 = b.shape[1]
    I = N2 // 2
    dev = a.device
    _dev(a, "a", dev)
    _need(b, "b", b.dtype, (G, N2, K), dev)
    _need(a_sf, "a_sf", torch.float32, (G, M_max, K // BLOCK), dev)
    _need(b_sf, "b_sf", torch.float32, (G, N2 // BLOCK, K // BLOCK), dev)
    _need(masked_m, "masked_m", torch.int32, (G,), dev)
    codes, sf = _swiglu_outputs((G, M_max), I, codes, sf, dev)
    _run(dev, lib.dg_m_grouped_fp8_gemm_nt_masked_swiglu, a.data_ptr(), b.data_ptr(),
         codes.data_ptr(), sf.data_ptr(), a_sf.data_ptr(), b_sf.data_ptr(), masked_m.data_ptr(),
         G, M_max, I, K)
    return codes, sf


def quantize_fp8_1x128(x, codes=None, sf=None):
    """Per-token 1x128 quantization of x [M, K] (float32 or bfloat16): returns
    (codes [M, K] torch.float8_e4m3fn, sf [M, K/128] torch.float32), written into the
    given tensors when passed (new tensors otherwise)."""
    if x.dim() != 2:
        raise ValueError("x must be [M, K]")
    if x.dtype == torch.float32:
        dtype = DTYPE_F32
    elif x.dtype == torch.bfloat16:
        dtype = DTYPE_BF16
    else:
        raise TypeError(f"x must be torch.float32 or torch.bfloat16, got {x.dtype}")
    M, K = x.shape
    dev = x.device
    _dev(x, "x", dev)
    if codes is None:
        codes = torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev)
    if sf is None:
        sf = torch.empty((M, K // BLOCK), dtype=torch.float32, device=dev)
    _fp8(codes, "codes")
    _need(codes, "codes", codes.dtype, (M, K), dev)
    _need(sf, "sf", torch.float32, (M, K // BLOCK), dev)
    _run(dev, lib.dg_quantize_fp8_1x128, x.data_ptr(), dtype, codes.data_ptr(), sf.data_ptr(),
         M, K)
    return codes, sf


def release_workspaces() -> None:
    """Free the library's own device buffers (split-K partials and counters, transposed
    operand copies) after the devices holding them go idle. No HIP graph holding a
    library call may be replayed afterwards."""
    check(lib.dg_release_workspaces())


def describe_config(kind: int, M: int, N: int, K: int, G: int = 1, expected_m: int = 0) -> str:
    buf = ctypes.create_string_buffer(128)
    check(lib.dg_describe_config(kind, M, N, K, G, expected_m, buf, 128))
    return buf.value.decode()


def config_names() -> list[str]:
    return [lib.dg_config_name(i).decode() for i in range(lib.dg_num_configs())]


__all__ = ["config_names", "fp8_gemm_nt", "fp8_gemm_nn", "fp8_gemm_tn", "fp8_gemm_tt", "m_grouped_fp8_gemm_nt_contiguous", "m_grouped_fp8_gemm_nt_masked",
           "m_grouped_fp8_gemm_nt_contiguous_swiglu", "m_grouped_fp8_gemm_nt_masked_swiglu",
           "quantize_fp8_1x128", "describe_config", "release_workspaces", "BUILD_ID", "DGError", "lib", "LIB_PATH"]
