"""GPU parity of the grouped GEMM with the fused SwiGLU + requantization epilogue
(dg_m_grouped_fp8_gemm_nt_{contiguous,masked}_swiglu) against the oracle: the exact
gate and up products (grouped oracle), h = silu(gate) * up in fp64 (oracle.swiglu),
and the oracle's quantizer.

The kernel forms h in fp32 from fp32 accumulators, so near a rounding boundary the
fp64 value may fall on the other side. The check is an interval one. With dh a bound
on |h_gpu - h|:
  * every scale 2^e lies between the scales of the smallest and largest block amax
    that h +- dh allows;
  * every code decodes to a value within dh + half an e4m3fn ulp (times the scale)
    of h;
  * where the interval leaves one choice, the code equals the oracle quantizer's
    (integer-valued inputs: all but the rare elements within 2^-19 of a midpoint).
dh: integer-valued operands make gate and up exact in fp32, leaving the fp32 SwiGLU
(2^-19 relative); for N(0,1) operands the GEMM's error reading (2e-3 of
max(|r|, rho/16)) bounds gate and up, propagated through silu (|silu'| <= 1.1).
Rows that are not produced keep their seeded bytes in both outputs.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu
from tests.test_gpu_parity import int_operands
from tests.test_gpu_quant import GuardedBytes

pytestmark = pytest.mark.gpu

E4M3 = oracle.e4m3fn_values()  # value of every code (NaN for 0x7F, 0xFF)


def half_ulp_e4m3(y):
    """Half the e4m3fn spacing at |y| (|y| <= 448): 2^(E-4) in [2^E, 2^(E+1)), E >= -6;
    2^-10 below 2^-6."""
    a = np.abs(y)
    E = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return np.ldexp(1.0, (E - 4).astype(int))


def run_swiglu(kind, A, B, sfA, sfB, idx, lead, I, seed=9):
    import fp8_block_scaled_dg_amd as dg
    rows = int(np.prod(lead))
    codes = GuardedBytes(rows * I, seed)
    sf = GuardedBytes(rows * (I // 128) * 4, seed + 1)
    gu.announce(f"swiglu {kind} rows={rows} I={I} K={A.shape[-1]}")
    fn = (dg.m_grouped_fp8_gemm_nt_contiguous_swiglu if kind == "contiguous"
          else dg.m_grouped_fp8_gemm_nt_masked_swiglu)
    fn(gu.codes(A), gu.codes(B), gu.dev(sfA), gu.dev(sfB), gu.dev(np.asarray(idx, np.int32)),
       codes.view(torch.float8_e4m3fn, lead + (I,)), sf.view(torch.float32, lead + (I // 128,)))
    torch.cuda.synchronize()
    assert codes.guards_intact() and sf.guards_intact(), "write outside the outputs"
    c = codes.result().reshape(rows, I)
    s = sf.result().view(np.float32).reshape(rows, I // 128)
    c0 = codes.host[4096:4096 + rows * I].reshape(rows, I)
    s0 = sf.host[4096:4096 + rows * (I // 128) * 4].view(np.float32).reshape(rows, I // 128)
    return c, s, c0, s0


def check(h, dh, codes, sf, what, strict):
    """h, dh [n][I] fp64; codes uint8 [n][I]; sf fp32 [n][I/128]."""
    n, I = h.shape
    hb, db = h.reshape(n, I // 128, 128), dh.reshape(n, I // 128, 128)
    sf64 = sf.astype(np.float64)
    m, x = np.frexp(sf64)
    assert np.all(m == 0.5), f"{what}: a scale is not a power of two"
    e_gpu = x - 1
    exp_of = np.vectorize(oracle.scale_exponent)
    e_lo = exp_of(np.max(np.maximum(np.abs(hb) - db, 0.0), axis=2))
    e_hi = exp_of(np.max(np.abs(hb) + db, axis=2))
    bad = np.nonzero((e_gpu < e_lo) | (e_gpu > e_hi))
    assert bad[0].size == 0, f"{what}: {bad[0].size} block scales outside the allowed range"
    s = np.repeat(sf64, 128, axis=1)
    q = E4M3[codes].astype(np.float64) * s
    assert not np.any(np.isnan(q)), f"{what}: NaN code"
    slack = dh + half_ulp_e4m3((np.abs(h) + dh) / s) * s
    err = np.abs(q - h)
    worst = np.max(err / slack)
    assert worst <= 1.0 + 1e-9, f"{what}: |dequant - h| reaches {worst:.3f} of the bound"
    # decisions against the oracle quantizer (h rounded to fp32, the kernel's precision)
    rc, rs = oracle.quantize_blocks(h.astype(np.float32), 1, 128)
    same_scale = np.repeat(rs == sf, 128, axis=1)
    match = (codes == rc) & same_scale
    frac = match.mean()
    if strict:
        lo = np.abs(h) - dh
        hi = np.abs(h) + dh
        y_lo, y_hi = lo / s, hi / s
        # one choice when both ends round to the same e4m3fn magnitude
        one = (lo > 0) & (oracle_nearest_mag(y_lo) == oracle_nearest_mag(y_hi))
        one &= np.repeat(e_lo == e_hi, 128, axis=1)
        assert np.all(match[one]), f"{what}: {np.sum(~match[one])} unambiguous codes differ"
    assert frac >= 0.99, f"{what}: only {frac:.4f} of codes match the oracle quantizer"
    return dict(n=int(h.size), code_match=float(frac), worst=float(worst))


_POS = E4M3[:127].astype(np.float64)  # finite non-negative values, ascending


def oracle_nearest_mag(y):
    """Index of the e4m3fn magnitude nearest to |y| (ties to the even code), |y| <= 448."""
    a = np.minimum(np.abs(y), 448.0)
    i = np.clip(np.searchsorted(_POS, a), 1, 126)
    lo, hi = _POS[i - 1], _POS[i]
    pick_hi = (a - lo > hi - a) | ((a - lo == hi - a) & ((i % 2) == 0))
    return np.where(pick_hi, i, i - 1)


def exact_dh(h):
    return np.abs(h) * 2.0 ** -19 + 1e-300


def gemm_dh(g, u):
    """dh for N(0,1) operands from the GEMM error reading on gate and up."""
    rho = np.sqrt(np.mean(np.concatenate([g.ravel(), u.ravel()]) ** 2))
    dg_ = 2e-3 * np.maximum(np.abs(g), rho / 16)
    du = 2e-3 * np.maximum(np.abs(u), rho / 16)
    sil = np.abs(g / (1 + np.exp(-np.clip(g, -700, 700))))
    h = sil * np.abs(u)
    return 1.1 * np.abs(u) * dg_ + sil * du + 1.1 * dg_ * du + h * 2.0 ** -19 + 1e-300


def test_contiguous_small_integer_exact():
    rng = np.random.default_rng(51)
    G, I, K = 4, 256, 384
    counts = np.array([5, 0, 130, 64], dtype=np.int32)
    m_indices = synth.contiguous_layout(counts)
    A, B, sfA, sfB = int_operands(rng, m_indices.size, 2 * I, K, G=G)
    c, s, c0, s0 = run_swiglu("contiguous", A, B, sfA, sfB, m_indices, (m_indices.size,), I)
    gu_, produced = oracle.grouped_contiguous(A, B, sfA, sfB, m_indices)
    h = oracle.swiglu(gu_[produced])
    print(check(h, exact_dh(h), c[produced], s[produced], "contiguous int", strict=True))
    assert np.array_equal(c[~produced], c0[~produced]) and np.array_equal(
        s[~produced].view(np.uint32), s0[~produced].view(np.uint32)), "pad rows written"


def test_contiguous_unaligned_mixed_ids_integer_exact():
    rng = np.random.default_rng(52)
    G, I, K, M_total = 5, 128, 256, 300
    m_indices = rng.integers(-2, G + 2, size=M_total).astype(np.int32)
    m_indices[:40] = 3
    A, B, sfA, sfB = int_operands(rng, M_total, 2 * I, K, G=G)
    c, s, c0, s0 = run_swiglu("contiguous", A, B, sfA, sfB, m_indices, (M_total,), I)
    gu_, produced = oracle.grouped_contiguous(A, B, sfA, sfB, m_indices)
    h = oracle.swiglu(gu_[produced])
    print(check(h, exact_dh(h), c[produced], s[produced], "contiguous mixed", strict=True))
    assert np.array_equal(c[~produced], c0[~produced])


def test_masked_small_integer_exact():
    rng = np.random.default_rng(53)
    G, M_max, I, K = 3, 150, 384, 256
    A, B, sfA, sfB = int_operands(rng, G * M_max, 2 * I, K, G=G)
    A, sfA = A.reshape(G, M_max, K), sfA.reshape(G, M_max, K // 128)
    masked_m = np.array([150, 0, 77], dtype=np.int32)
    c, s, c0, s0 = run_swiglu("masked", A, B, sfA, sfB, masked_m, (G, M_max), I)
    gu_, produced = oracle.grouped_masked(A, B, sfA, sfB, masked_m)
    p = produced.ravel()
    h = oracle.swiglu(gu_.reshape(G * M_max, 2 * I)[p])
    print(check(h, exact_dh(h), c[p], s[p], "masked int", strict=True))
    assert np.array_equal(c[~p], c0[~p]) and np.array_equal(s[~p].view(np.uint32),
                                                            s0[~p].view(np.uint32))


def test_contiguous_gaussian_nan_pad():
    counts = np.array([3, 130, 0, 64], dtype=np.int32)
    w = synth.contiguous(4, 512, 512, 0, seed_base=889100, counts=counts,
                         pad_code=synth.FP8_NAN_CODE)
    M_total, N2, K, G = w.shape
    c, s, c0, s0 = run_swiglu("contiguous", w.A, w.B, w.sfA, w.sfB, w.m_indices, (M_total,), N2 // 2)
    gu_, produced = oracle.grouped_contiguous(w.A, w.B, w.sfA, w.sfB, w.m_indices)
    g, u = gu_[produced][:, :N2 // 2], gu_[produced][:, N2 // 2:]
    h = oracle.swiglu(gu_[produced])
    print(check(h, gemm_dh(g, u), c[produced], s[produced], "contiguous N(0,1)", strict=False))
    assert np.array_equal(c[~produced], c0[~produced])


def test_contiguous_workload_sampled():
    # the MoE contiguous workload read as Linear1 of a layer with I = 2048:
    # B [32][4096][7168] = [gate; up]
    w = synth.workload("moe_cont")
    M_total, N2, K, G = w.shape
    I = N2 // 2
    c, s, _, _ = run_swiglu("contiguous", w.A, w.B, w.sfA, w.sfB, w.m_indices, (M_total,), I)
    rng = np.random.default_rng(54)
    real = np.nonzero(w.m_indices >= 0)[0]
    firsts = [np.nonzero(w.m_indices == e)[0] for e in range(G) if w.counts[e] > 0]
    rows = np.unique(np.concatenate([rng.choice(real, 48, replace=False),
                                     [f[0] for f in firsts], [f[-1] for f in firsts]]))
    ri = np.repeat(rows, N2).astype(np.int64)
    ni = np.tile(np.arange(N2, dtype=np.int64), rows.size)
    gu_ = oracle.grouped_contiguous_at(w.A, w.B, w.sfA, w.sfB, w.m_indices, ri, ni)
    gu_ = gu_.reshape(rows.size, N2)
    h = oracle.swiglu(gu_)
    print(check(h, gemm_dh(gu_[:, :I], gu_[:, I:]), c[rows], s[rows], "moe_cont swiglu",
                strict=False))


def test_masked_workload_sampled():
    # the MoE masked workload read as Linear1 with I = 3584: B [32][7168][2048]
    w = synth.workload("moe_mask", pad_code=synth.FP8_NAN_CODE)
    G, M_max, N2, K = w.shape
    I = N2 // 2
    c, s, c0, s0 = run_swiglu("masked", w.A, w.B, w.sfA, w.sfB, w.masked_m, (G, M_max), I)
    produced = (np.arange(M_max)[None, :] < np.clip(w.masked_m, 0, M_max)[:, None]).ravel()
    assert np.array_equal(c[~produced], c0[~produced]), "masked rows written"
    rng = np.random.default_rng(55)
    rows = np.sort(rng.choice(np.nonzero(produced)[0], 64, replace=False))
    ri = np.repeat(rows, N2).astype(np.int64)
    ni = np.tile(np.arange(N2, dtype=np.int64), rows.size)
    gu_ = oracle.grouped_masked_at(w.A, w.B, w.sfA, w.sfB, w.masked_m, ri // M_max, ri % M_max, ni)
    gu_ = gu_.reshape(rows.size, N2)
    h = oracle.swiglu(gu_)
    print(check(h, gemm_dh(gu_[:, :I], gu_[:, I:]), c[rows], s[rows], "moe_mask swiglu",
                strict=False))
