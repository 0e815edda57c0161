"""Seeded synthetic inputs for the FP8 block-scaled GEMM workloads.

This package only makes inputs; both the GPU library's tests and benchmark and the
CPU oracle's tests consume what it writes. It contains none of the GEMM arithmetic
and imports neither the library nor the oracle. The recipe is stated in
``dg_synth.cpp``; the workloads are:

========  ===================================================================
name      shape
========  ===================================================================
small     dense NT  M=128  N=256   K=512
dec2112   dense NT  M=64   N=2112  K=7168     (decode, memory-bound)
dec32768  dense NT  M=64   N=32768 K=512      (decode, memory-bound)
prefill   dense NT  M=4096 N=7168  K=18432    (compute-bound)
moe_cont  grouped contiguous: 32 experts, N=4096, K=7168, 8192 tokens routed by
          Zipf(1.1) over 28 experts (4 seeded experts empty), segments padded to
          multiples of 128 rows, pad rows have m_index = -1
moe_mask  grouped masked: 32 experts, M_max=256, N=7168, K=2048,
          masked_m[e] uniform on {0..256}
========  ===================================================================

Seeds: each workload has an index w (small=0, dec2112=1, dec32768=2, prefill=3,
moe_cont=4, moe_mask=5); stream seeds are 1000*w + role with role 1 = A, 2 = B,
3 = routing counts or masked_m, 4 = expert permutation.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdg_synth.so")
SOURCE_PATH = os.path.join(_HERE, "dg_synth.cpp")

BLOCK = 128
FP8_NAN_CODE = 0x7F

ROLE_A, ROLE_B, ROLE_ROUTE, ROLE_PERM = 1, 2, 3, 4

_lib = None
_u8p = ctypes.POINTER(ctypes.c_uint8)
_f32p = ctypes.POINTER(ctypes.c_float)
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64 = ctypes.c_int64
_u64 = ctypes.c_uint64


def build_command() -> list[str]:
    return ["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
            "-o", LIB_PATH, SOURCE_PATH]


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SOURCE_PATH):
        subprocess.run(build_command(), check=True)
    lib = ctypes.CDLL(LIB_PATH)
    lib.dgs_mt_output.restype = ctypes.c_uint64
    lib.dgs_mt_output.argtypes = [_u64, _i64]
    lib.dgs_normal_rows.argtypes = [_u64, _i64, _i64, _f32p]
    lib.dgs_quantize.argtypes = [_f32p, _i64, _i64, _i64, _i64, _u8p, _f32p]
    lib.dgs_make_operand.argtypes = [_u64, _i64, _i64, _i64, _i64, _u8p, _f32p]
    lib.dgs_permutation.argtypes = [_u64, ctypes.c_int32, _i32p]
    lib.dgs_zipf_counts.argtypes = [_u64, _i64, ctypes.c_int32, ctypes.c_double, _i32p]
    lib.dgs_uniform_ints.argtypes = [_u64, _i64, _i64, _i32p]
    _lib = lib
    return lib


def _p(a, t):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(t)


def mt_output(seed: int, index: int) -> int:
    return int(_load().dgs_mt_output(seed, index))


def normal_rows(seed: int, R: int, C: int) -> np.ndarray:
    out = np.empty((R, C), dtype=np.float32)
    _load().dgs_normal_rows(seed, R, C, _p(out, _f32p))
    return out


def quantize(x: np.ndarray, br: int, bc: int = BLOCK):
    """(codes uint8 [R][C], scales fp32 [ceil(R/br)][C/bc]) of fp32 x [R][C]."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, C = x.shape
    assert C % bc == 0
    codes = np.empty((R, C), dtype=np.uint8)
    scales = np.empty(((R + br - 1) // br, C // bc), dtype=np.float32)
    _load().dgs_quantize(_p(x, _f32p), R, C, br, bc, _p(codes, _u8p), _p(scales, _f32p))
    return codes, scales


def pack_ue8m0(sf: np.ndarray) -> np.ndarray:
    """The packed UE8M0 form of power-of-two scales sf [..., KB]: int32 [..., ceil(KB/4)]
    words whose byte j (little-endian) of word w is e + 127 for the scale 2^e of
    K-block 4w + j; padding bytes are 0. An input layout, not arithmetic of the method."""
    sf = np.asarray(sf, dtype=np.float32)
    m, e = np.frexp(sf.astype(np.float64))
    if not np.all(m == 0.5):
        raise ValueError("UE8M0 holds powers of two only")
    b = e - 1 + 127
    if b.size and (b.min() < 0 or b.max() > 254):
        raise ValueError("scale exponent outside the UE8M0 range")
    KB = sf.shape[-1]
    words = (KB + 3) // 4
    out = np.zeros(sf.shape[:-1] + (words * 4,), dtype=np.uint8)
    out[..., :KB] = b
    return np.ascontiguousarray(out).view("<i4").reshape(sf.shape[:-1] + (words,))


def make_operand(seed: int, R: int, C: int, br: int):
    """Draw N(0,1) R x C (as normal_rows(seed, R, C)) and quantize with br x 128 blocks."""
    assert C % BLOCK == 0 and br in (1, BLOCK)
    codes = np.empty((R, C), dtype=np.uint8)
    scales = np.empty(((R + br - 1) // br, C // BLOCK), dtype=np.float32)
    if R > 0:
        _load().dgs_make_operand(seed, R, C, br, BLOCK, _p(codes, _u8p), _p(scales, _f32p))
    return codes, scales


def permutation(seed: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().dgs_permutation(seed, n, _p(out, _i32p))
    return out


def zipf_counts(seed: int, n_tokens: int, n_ranks: int, s: float) -> np.ndarray:
    out = np.empty(n_ranks, dtype=np.int32)
    _load().dgs_zipf_counts(seed, n_tokens, n_ranks, s, _p(out, _i32p))
    return out


def uniform_ints(seed: int, n: int, bound: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().dgs_uniform_ints(seed, n, bound, _p(out, _i32p))
    return out


# ----------------------------------------------------------------- workloads


@dataclasses.dataclass
class Dense:
    A: np.ndarray    # uint8 e4m3fn codes [M][K]
    sfA: np.ndarray  # fp32 [M][K/128]
    B: np.ndarray    # uint8 [N][K]
    sfB: np.ndarray  # fp32 [ceil(N/128)][K/128]

    @property
    def shape(self):
        return self.A.shape[0], self.B.shape[0], self.A.shape[1]


@dataclasses.dataclass
class Contiguous:
    A: np.ndarray          # uint8 [M_total][K]
    sfA: np.ndarray        # fp32 [M_total][K/128]
    B: np.ndarray          # uint8 [G][N][K]
    sfB: np.ndarray        # fp32 [G][ceil(N/128)][K/128]
    m_indices: np.ndarray  # int32 [M_total], -1 on pad rows
    counts: np.ndarray     # int32 [G] real rows per expert

    @property
    def shape(self):
        G, N, K = self.B.shape
        return self.A.shape[0], N, K, G


@dataclasses.dataclass
class Masked:
    A: np.ndarray         # uint8 [G][M_max][K]
    sfA: np.ndarray       # fp32 [G][M_max][K/128]
    B: np.ndarray         # uint8 [G][N][K]
    sfB: np.ndarray       # fp32 [G][ceil(N/128)][K/128]
    masked_m: np.ndarray  # int32 [G]

    @property
    def shape(self):
        G, M_max, K = self.A.shape
        return G, M_max, self.B.shape[1], K


def dense(M: int, N: int, K: int, seed_base: int) -> Dense:
    A, sfA = make_operand(seed_base + ROLE_A, M, K, 1)
    B, sfB = make_operand(seed_base + ROLE_B, N, K, BLOCK)
    return Dense(A, sfA, B, sfB)


def grouped_weights(G: int, N: int, K: int, seed_base: int):
    """B [G][N][K] and sfB [G][ceil(N/128)][K/128]; expert e from seed (base+2)*1024+e."""
    NB, KB = (N + BLOCK - 1) // BLOCK, K // BLOCK
    B = np.empty((G, N, K), dtype=np.uint8)
    sfB = np.empty((G, NB, KB), dtype=np.float32)
    for e in range(G):
        B[e], sfB[e] = make_operand((seed_base + ROLE_B) * 1024 + e, N, K, BLOCK)
    return B, sfB


def contiguous_layout(counts: np.ndarray, align: int = BLOCK) -> np.ndarray:
    """m_indices for segments in expert-id order, each padded to a multiple of align."""
    parts = []
    for e, c in enumerate(counts.tolist()):
        if c == 0:
            continue
        padded = -(-c // align) * align
        seg = np.full(padded, -1, dtype=np.int32)
        seg[:c] = e
        parts.append(seg)
    return np.concatenate(parts) if parts else np.zeros(0, dtype=np.int32)


def contiguous(G: int, N: int, K: int, n_tokens: int, seed_base: int, zipf_s: float = 1.1,
               n_empty: int = 4, counts: np.ndarray | None = None,
               pad_code: int = 0) -> Contiguous:
    """Zipf-routed contiguous MoE inputs. `counts` overrides the routing draw."""
    if counts is None:
        ranks = zipf_counts(seed_base + ROLE_ROUTE, n_tokens, G - n_empty, zipf_s)
        perm = permutation(seed_base + ROLE_PERM, G)
        counts = np.zeros(G, dtype=np.int32)
        counts[perm[: G - n_empty]] = ranks
    counts = np.asarray(counts, dtype=np.int32)
    m_indices = contiguous_layout(counts)
    M_total = m_indices.shape[0]
    tok_codes, tok_sf = make_operand(seed_base + ROLE_A, int(counts.sum()), K, 1)
    A = np.full((M_total, K), pad_code, dtype=np.uint8)
    sfA = np.ones((M_total, K // BLOCK), dtype=np.float32)
    real = m_indices >= 0
    A[real] = tok_codes
    sfA[real] = tok_sf
    B, sfB = grouped_weights(G, N, K, seed_base)
    return Contiguous(A, sfA, B, sfB, m_indices, counts)


def masked(G: int, M_max: int, N: int, K: int, seed_base: int,
           masked_m: np.ndarray | None = None, pad_code: int = 0) -> Masked:
    """Masked MoE inputs; rows m >= masked_m[e] hold pad_code with scale 1."""
    if masked_m is None:
        masked_m = uniform_ints(seed_base + ROLE_ROUTE, G, M_max + 1)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    codes, sf = make_operand(seed_base + ROLE_A, G * M_max, K, 1)
    A = codes.reshape(G, M_max, K)
    sfA = sf.reshape(G, M_max, K // BLOCK)
    rows = np.arange(M_max)[None, :] >= np.clip(masked_m, 0, M_max)[:, None]
    A[rows] = pad_code
    sfA[rows] = 1.0
    B, sfB = grouped_weights(G, N, K, seed_base)
    return Masked(A, sfA, B, sfB, masked_m)


WORKLOADS = {
    "small": dict(kind="dense", index=0, M=128, N=256, K=512),
    "dec2112": dict(kind="dense", index=1, M=64, N=2112, K=7168),
    "dec32768": dict(kind="dense", index=2, M=64, N=32768, K=512),
    "prefill": dict(kind="dense", index=3, M=4096, N=7168, K=18432),
    "moe_cont": dict(kind="contiguous", index=4, G=32, N=4096, K=7168, tokens=8192),
    "moe_mask": dict(kind="masked", index=5, G=32, M_max=256, N=7168, K=2048),
}


def workload(name: str, pad_code: int = 0):
    w = WORKLOADS[name]
    base = 1000 * w["index"]
    if w["kind"] == "dense":
        return dense(w["M"], w["N"], w["K"], base)
    if w["kind"] == "contiguous":
        return contiguous(w["G"], w["N"], w["K"], w["tokens"], base, pad_code=pad_code)
    return masked(w["G"], w["M_max"], w["N"], w["K"], base, pad_code=pad_code)
