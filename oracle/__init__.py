"""CPU oracle for the FP8 block-scaled GEMM -- TEST INFRASTRUCTURE.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may import
this package. The product library never calls it and shares no code with it.

It wraps ``dg_oracle.c`` (plain C, fp64) through ctypes. What each function computes,
and the passages of the pages it follows, are stated in that file:

* ``gemm_nt`` / ``gemm_nt_at``: the dense block-scaled product
  C = sum_kb sfA * sfB * dot(fp8 block) -- DeepGEMM launch article (deepseek.csdn.net),
  section 1.2 "precision safeguards" (per-block scaling factors, FP32 promotion);
  DeepGEMM project page (aiproducthub.cn), "quick start" (call shape).
* ``grouped_contiguous`` / ``grouped_contiguous_at``: MoE rows concatenated along M
  with a per-row expert id -- project page, "technical implementation".
* ``grouped_masked`` / ``grouped_masked_at``: per-expert slab with a valid-row count
  -- launch article section 4.2 "advanced tuning"; library news page (youleyou.com),
  "performance".
* ``quantize_blocks``: power-of-two per-block scale and nearest-e4m3fn codes, written
  as a search (launch article section 1.2).
* ``bf16_rne``: one rounding from fp64 to bf16.
* ``gemm``: the dense product in the NT / NN / TN / TT memory layouts -- project
  page, "core features".
* ``swiglu``: h = silu(gate) * up between the two grouped GEMMs of an MoE layer --
  project page, "core features" (Mega MoE: Linear1, SwiGLU, Linear2 fused).
* ``unpack_ue8m0``: fp32 scales from the packed exponent-byte (UE8M0) layout of the
  LHS scaling factors -- project page, "technical implementation".

Every function here is pinned by CPU tests against values fixed by the format
definitions and by closed forms (``tests/test_oracle_*.py``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg_oracle.so")
SOURCE_PATH = os.path.join(_HERE, "dg_oracle.c")

_lib = None

_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_u16p = ctypes.POINTER(ctypes.c_uint16)
_i64 = ctypes.c_int64


def build_command() -> list[str]:
    """gcc line that builds the oracle library (no fast-math, no FMA contraction)."""
    return ["gcc", "-O2", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
            "-shared", "-fPIC", "-o", LIB_PATH, SOURCE_PATH, "-lm"]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE_PATH):
        import subprocess
        subprocess.run(build_command(), check=True)
    lib = ctypes.CDLL(LIB_PATH)
    lib.dgo_e4m3fn_value.restype = ctypes.c_double
    lib.dgo_e4m3fn_value.argtypes = [ctypes.c_uint8]
    lib.dgo_bf16_rne.restype = ctypes.c_uint16
    lib.dgo_bf16_rne.argtypes = [ctypes.c_double]
    lib.dgo_bf16_rne_array.argtypes = [_f64p, _u16p, _i64]
    lib.dgo_gemm_nt.argtypes = [_u8p, _u8p, _f32p, _f32p, _i64, _i64, _i64, _f64p]
    lib.dgo_gemm_nt_at.argtypes = [_u8p, _u8p, _f32p, _f32p, _i64, _i64, _i64,
                                   _i64p, _i64p, _i64, _f64p]
    lib.dgo_grouped_contiguous.argtypes = [_u8p, _u8p, _f32p, _f32p, _i32p, _i64, _i64,
                                           _i64, ctypes.c_int32, _f64p, _u8p]
    lib.dgo_grouped_contiguous_at.argtypes = [_u8p, _u8p, _f32p, _f32p, _i32p, _i64, _i64,
                                              _i64, ctypes.c_int32, _i64p, _i64p, _i64, _f64p]
    lib.dgo_grouped_masked.argtypes = [_u8p, _u8p, _f32p, _f32p, _i32p, ctypes.c_int32,
                                       _i64, _i64, _i64, _f64p, _u8p]
    lib.dgo_grouped_masked_at.argtypes = [_u8p, _u8p, _f32p, _f32p, _i32p, ctypes.c_int32,
                                          _i64, _i64, _i64, _i64p, _i64p, _i64p, _i64, _f64p]
    lib.dgo_scale_exponent.restype = ctypes.c_int
    lib.dgo_scale_exponent.argtypes = [ctypes.c_double]
    lib.dgo_e4m3fn_nearest.restype = ctypes.c_uint8
    lib.dgo_e4m3fn_nearest.argtypes = [ctypes.c_double]
    lib.dgo_quantize_blocks.argtypes = [_f32p, _i64, _i64, _i64, _i64, _u8p, _f32p]
    lib.dgo_gemm_layout.argtypes = [_u8p, _u8p, _f32p, _f32p, _i64, _i64, _i64, ctypes.c_int,
                                    ctypes.c_int, _f64p]
    lib.dgo_swiglu.argtypes = [_f64p, _i64, _i64, _f64p]
    lib.dgo_unpack_ue8m0.argtypes = [ctypes.POINTER(ctypes.c_uint32), _i64, _i64, _f32p]
    lib.dgo_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _p(arr: np.ndarray, ptype):
    assert arr.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return arr.ctypes.data_as(ptype)


def _codes(x) -> np.ndarray:
    x = np.ascontiguousarray(x)
    return x.view(np.uint8) if x.dtype != np.uint8 else x


def num_threads() -> int:
    return int(_load().dgo_num_threads())


def e4m3fn_value(code: int) -> float:
    return float(_load().dgo_e4m3fn_value(int(code) & 0xFF))


def e4m3fn_values() -> np.ndarray:
    """fp64 value of every code 0..255 (NaN for 0x7F and 0xFF)."""
    return np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)


def bf16_rne(x) -> np.ndarray:
    """bf16 bit patterns (uint16) of fp64 values, one RNE rounding."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty(x.shape, dtype=np.uint16)
    _load().dgo_bf16_rne_array(_p(x, _f64p), _p(out, _u16p), x.size)
    return out


def gemm_nt(A, B, sfA, sfB) -> np.ndarray:
    """fp64 C [M][N] of the dense block-scaled NT product."""
    A, B = _codes(A), _codes(B)
    sfA = np.ascontiguousarray(sfA, dtype=np.float32)
    sfB = np.ascontiguousarray(sfB, dtype=np.float32)
    M, K = A.shape
    N = B.shape[0]
    C = np.empty((M, N), dtype=np.float64)
    _load().dgo_gemm_nt(_p(A, _u8p), _p(B, _u8p), _p(sfA, _f32p), _p(sfB, _f32p), M, N, K,
                        _p(C, _f64p))
    return C


def gemm_nt_at(A, B, sfA, sfB, m_idx, n_idx) -> np.ndarray:
    A, B = _codes(A), _codes(B)
    sfA = np.ascontiguousarray(sfA, dtype=np.float32)
    sfB = np.ascontiguousarray(sfB, dtype=np.float32)
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    M, K = A.shape
    N = B.shape[0]
    out = np.empty(m_idx.shape, dtype=np.float64)
    _load().dgo_gemm_nt_at(_p(A, _u8p), _p(B, _u8p), _p(sfA, _f32p), _p(sfB, _f32p), M, N, K,
                           _p(m_idx, _i64p), _p(n_idx, _i64p), m_idx.size, _p(out, _f64p))
    return out


def grouped_contiguous(A, B, sfA, sfB, m_indices):
    """(C_exact [M_total][N] with NaN in rows not produced, produced [M_total] bool)."""
    A, B = _codes(A), _codes(B)
    sfA = np.ascontiguousarray(sfA, dtype=np.float32)
    sfB = np.ascontiguousarray(sfB, dtype=np.float32)
    m_indices = np.ascontiguousarray(m_indices, dtype=np.int32)
    M_total, K = A.shape
    G, N, _ = B.shape
    C = np.full((M_total, N), np.nan, dtype=np.float64)
    produced = np.zeros(M_total, dtype=np.uint8)
    _load().dgo_grouped_contiguous(_p(A, _u8p), _p(B, _u8p), _p(sfA, _f32p), _p(sfB, _f32p),
                                   _p(m_indices, _i32p), M_total, N, K, G, _p(C, _f64p),
                                   _p(produced, _u8p))
    return C, produced.astype(bool)


def grouped_contiguous_at(A, B, sfA, sfB, m_indices, r_idx, n_idx) -> np.ndarray:
    A, B = _codes(A), _codes(B)
    sfA = np.ascontiguousarray(sfA, dtype=np.float32)
    sfB = np.ascontiguousarray(sfB, dtype=np.float32)
    m_indices = np.ascontiguousarray(m_indices, dtype=np.int32)
    r_idx = np.ascontiguousarray(r_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    M_total, K = A.shape
    G, N, _ = B.shape
    out = np.empty(r_idx.shape, dtype=np.float64)
    _load().dgo_grouped_contiguous_at(_p(A, _u8p), _p(B, _u8p), _p(sfA, _f32p), _p(sfB, _f32p),
                                      _p(m_indices, _i32p), M_total, N, K, G, _p(r_idx, _i64p),
                                      _p(n_idx, _i64p), r_idx.size, _p(out, _f64p))
    return out


def grouped_masked(A, B, sfA, sfB, masked_m):
    """(C_exact [G][M_max][N] with NaN in rows not produced, produced [G][M_max] bool)."""
    A, B = _codes(A), _codes(B)
    sfA = np.ascontiguousarray(sfA, dtype=np.float32)
    sfB = np.ascontiguousarray(sfB, dtype=np.float32)
    masked_m = np.ascontiguousarray(masked_m, dtype=np.int32)
    G, M_max, K = A.shape
    N = B.shape[1]
    C = np.full((G, M_max, N), np.nan, dtype=np.float64)
    produced = np.zeros((G, M_max), dtype=np.uint8)
    _load().dgo_grouped_masked(_p(A, _u8p), _p(B, _u8p), _p(sfA, _f32p), _p(sfB, _f32p),
                               _p(masked_m, _i32p), G, M_max, N, K, _p(C, _f64p),
                               _p(produced, _u8p))
    return C, produced.astype(bool)


def grouped_masked_at(A, B, sfA, sfB, masked_m, e_idx, m_idx, n_idx) -> np.ndarray:
    A, B = _codes(A), _codes(B)
    sfA = np.ascontiguousarray(sfA, dtype=np.float32)
    sfB = np.ascontiguousarray(sfB, dtype=np.float32)
    masked_m = np.ascontiguousarray(masked_m, dtype=np.int32)
    e_idx = np.ascontiguousarray(e_idx, dtype=np.int64)
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    G, M_max, K = A.shape
    N = B.shape[1]
    out = np.empty(e_idx.shape, dtype=np.float64)
    _load().dgo_grouped_masked_at(_p(A, _u8p), _p(B, _u8p), _p(sfA, _f32p), _p(sfB, _f32p),
                                  _p(masked_m, _i32p), G, M_max, N, K, _p(e_idx, _i64p),
                                  _p(m_idx, _i64p), _p(n_idx, _i64p), e_idx.size,
                                  _p(out, _f64p))
    return out


def scale_exponent(amax: float) -> int:
    return int(_load().dgo_scale_exponent(float(amax)))


def e4m3fn_nearest(y: float) -> int:
    return int(_load().dgo_e4m3fn_nearest(float(y)))


def gemm(A, B, sfA, sfB, layout: str = "nt") -> np.ndarray:
    """C_exact [M][N] of C = op(A) op(B), layout "nt" | "nn" | "tn" | "tt": A stored
    [M][K] (first letter n) or [K][M] (t); B stored [K][N] (second letter n) or [N][K] (t)."""
    assert layout in ("nt", "nn", "tn", "tt")
    a_t, b_n = layout[0] == "t", layout[1] == "n"
    A, B = _codes(A), _codes(B)
    sfA = np.ascontiguousarray(sfA, dtype=np.float32)
    sfB = np.ascontiguousarray(sfB, dtype=np.float32)
    M = A.shape[1] if a_t else A.shape[0]
    K = A.shape[0] if a_t else A.shape[1]
    N = B.shape[1] if b_n else B.shape[0]
    assert (B.shape[0] if b_n else B.shape[1]) == K
    C = np.empty((M, N), dtype=np.float64)
    _load().dgo_gemm_layout(_p(A, _u8p), _p(B, _u8p), _p(sfA, _f32p), _p(sfB, _f32p), M, N, K,
                            int(a_t), int(b_n), _p(C, _f64p))
    return C


def swiglu(gu) -> np.ndarray:
    """h [..., I] = silu(gate) * up in fp64 from gu [..., 2I] (gate = first half)."""
    gu = np.ascontiguousarray(gu, dtype=np.float64)
    lead, two_i = gu.shape[:-1], gu.shape[-1]
    assert two_i % 2 == 0
    rows = int(np.prod(lead)) if lead else 1
    h = np.empty(lead + (two_i // 2,), dtype=np.float64)
    _load().dgo_swiglu(_p(gu, _f64p), rows, two_i // 2, _p(h, _f64p))
    return h


def unpack_ue8m0(packed, KB: int) -> np.ndarray:
    """fp32 scales [..., KB] from packed UE8M0 words [..., ceil(KB/4)] (uint32 or int32)."""
    packed = np.ascontiguousarray(packed).view(np.uint32)
    lead = packed.shape[:-1]
    assert packed.shape[-1] == (KB + 3) // 4
    rows = int(np.prod(lead)) if lead else 1
    out = np.empty(lead + (KB,), dtype=np.float32)
    _load().dgo_unpack_ue8m0(packed.ctypes.data_as(ctypes.POINTER(ctypes.c_uint32)), rows, KB,
                             _p(out, _f32p))
    return out


def quantize_blocks(x, br: int, bc: int):
    """(codes uint8 [R][C], scales fp32 [ceil(R/br)][C/bc]) for fp32 x [R][C]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % bc == 0
    codes = np.empty((R, C), dtype=np.uint8)
    scales = np.empty(((R + br - 1) // br, C // bc), dtype=np.float32)
    _load().dgo_quantize_blocks(_p(x, _f32p), R, C, br, bc, _p(codes, _u8p), _p(scales, _f32p))
    return codes, scales
