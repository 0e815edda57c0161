"""CPU pins for the oracle's format rules: e4m3fn decode, bf16 rounding, the block
quantizer. Each is checked against something other than the oracle itself: torch's
conversions (independent library routines), exact rational rounding, the OCP code
points in tests/golden, and closed-form invariants."""
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from tests import _exact

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_e4m3fn_decode_matches_torch_on_all_codes():
    ours = oracle.e4m3fn_values()
    ref = _exact.fp8_values_torch()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(ref[~nan]))


def test_e4m3fn_decode_golden_code_points():
    with open(os.path.join(GOLDEN, "e4m3fn_points.txt")) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    assert len(rows) >= 10
    for code_hex, value, *_ in rows:
        got = oracle.e4m3fn_value(int(code_hex, 16))
        if value == "nan":
            assert math.isnan(got)
        else:
            assert got == float(value) and math.copysign(1, got) == math.copysign(1, float(value))


def test_e4m3fn_values_monotone_and_nan_count():
    vals = oracle.e4m3fn_values()
    pos = vals[:127]
    assert np.all(np.diff(pos) > 0)  # codes 0..126 increase strictly
    assert np.isnan(vals).sum() == 2
    assert np.array_equal(vals[128:255], -pos)


def test_bf16_rne_exhaustive_fp32_binades_vs_torch():
    # every fp32 pattern in a few binades (normal, near subnormal, large), plus the
    # subnormal range edge: torch's fp32 -> bf16 conversion rounds to nearest even.
    pats = []
    for exp in (1, 2, 100, 127, 130, 253, 254):
        pats.append(np.arange(exp << 23, (exp + 1) << 23, 997, dtype=np.uint32))
    pats.append(np.arange(0, 1 << 23, 613, dtype=np.uint32))  # fp32 subnormals
    pats = np.concatenate(pats)
    pats = np.concatenate([pats, pats | 0x80000000])
    f32 = pats.view(np.float32)
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(f32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_bf16_rne_ties_vs_torch():
    # every tie: low 16 bits exactly 0x8000, for all high patterns of a binade span
    hi = np.arange(0x3F00, 0x4100, dtype=np.uint32)
    pats = (hi << 16) | 0x8000
    f32 = pats.view(np.float32)
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne(f32.astype(np.float64)), ref)


def test_bf16_rne_from_fp64_vs_exact_rational():
    rng = random.Random(7)
    xs = []
    for _ in range(400):
        xs.append(rng.uniform(-1e4, 1e4) * 2.0 ** rng.randint(-140, 120))
    # midpoints of bf16 neighbours, and one fp64 ulp either side (fp32 cannot hold these)
    for _ in range(300):
        hi = rng.randint(0x0001, 0x7F7E)
        lo = (np.array([hi << 16], dtype=np.uint32).view(np.float32)[0]).astype(np.float64)
        up = (np.array([(hi + 1) << 16], dtype=np.uint32).view(np.float32)[0]).astype(np.float64)
        mid = (lo + up) / 2
        xs += [mid, math.nextafter(mid, math.inf), math.nextafter(mid, -math.inf), -mid]
    xs += [0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 3 * 2.0 ** -135, 3.3895313892515355e38,
           3.39e38, 1e39]
    got = oracle.bf16_rne(np.array(xs))
    for x, g in zip(xs, got):
        want = _exact.bf16_round_exact(Fraction(x))
        if x == 0.0:
            want = 0x8000 if math.copysign(1, x) < 0 else 0
        assert int(g) == want, (x, hex(int(g)), hex(want))


def test_nearest_code_vs_torch_on_all_midpoints():
    vals = oracle.e4m3fn_values()[:127]
    ys = list(vals) + list((vals[:-1] + vals[1:]) / 2)
    ys += [math.nextafter(y, math.inf) for y in ys] + [math.nextafter(y, -math.inf) for y in ys]
    ys = [y for y in ys if 0 <= y <= 448]
    ys = ys + [-y for y in ys]
    f = np.array(ys, dtype=np.float64)
    # torch converts from fp32; keep the probes that fp32 holds exactly
    f = f[f.astype(np.float32).astype(np.float64) == f]
    ref = torch.from_numpy(f.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3fn_nearest(y) for y in f], dtype=np.uint8)
    assert np.array_equal(got, ref)


def test_scale_exponent_definition():
    # least e with amax <= 448 * 2^e, checked by its two defining inequalities
    rng = np.random.default_rng(3)
    for amax in list(rng.lognormal(0, 6, 2000)) + [448.0, 449.0, 224.0, 224.0001, 1.0, 2.0 ** -140]:
        e = oracle.scale_exponent(amax)
        assert amax <= 448.0 * 2.0 ** e
        assert amax > 448.0 * 2.0 ** (e - 1)
    assert oracle.scale_exponent(0.0) == 0


def _check_quant_invariants(x, codes, scales, br, bc):
    vals = oracle.e4m3fn_values()
    R, C = x.shape
    for rb in range(scales.shape[0]):
        for cb in range(scales.shape[1]):
            blk = x[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc].astype(np.float64)
            s = float(scales[rb, cb])
            m, e = math.frexp(s)
            assert m == 0.5, "scale must be a power of two"
            amax = np.abs(blk).max()
            if amax == 0:
                assert s == 1.0
                continue
            assert 224 < amax / s <= 448
            deq = vals[codes[rb * br:(rb + 1) * br, cb * bc:(cb + 1) * bc]] * s
            y = blk / s
            # error at most half the e4m3fn spacing at |y| (2^-10 in the subnormal range)
            ay = np.abs(y)
            spacing = np.where(ay < 2.0 ** -6, 2.0 ** -9,
                               2.0 ** (np.floor(np.log2(np.maximum(ay, 2.0 ** -6))) - 3))
            assert np.all(np.abs(deq - blk) <= spacing / 2 * s + 0.0)


@pytest.mark.parametrize("br,R", [(1, 5), (128, 200)])
def test_quantizer_invariants(br, R):
    rng = np.random.default_rng(11)
    x = (rng.standard_normal((R, 256)) * rng.lognormal(0, 3, (R, 1))).astype(np.float32)
    x[0, :128] = 0.0  # an all-zero block when br == 1
    codes, scales = oracle.quantize_blocks(x, br, 128)
    _check_quant_invariants(x, codes, scales, br, 128)


def test_quantizer_scale_covariance_and_idempotence():
    rng = np.random.default_rng(12)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    codes, scales = oracle.quantize_blocks(x, 1, 128)
    for j in (-5, 3):
        c2, s2 = oracle.quantize_blocks(np.ldexp(x, j), 1, 128)
        assert np.array_equal(c2, codes)
        assert np.array_equal(s2, np.ldexp(scales, j))
    deq = (oracle.e4m3fn_values()[codes] * np.repeat(scales, 128, axis=1)).astype(np.float32)
    c3, s3 = oracle.quantize_blocks(deq, 1, 128)
    assert np.array_equal(c3, codes) and np.array_equal(s3, scales)


# ------------------------------------------------------------------ UE8M0 scale bytes


def test_ue8m0_unpack_every_byte():
    # byte b means 2^(b - 127): checked against numpy's ldexp and against the fp32 bit
    # layout (exponent field b for b >= 1, the subnormal 2^-127 = 0x00400000 for b = 0)
    KB = 255
    packed = np.zeros((1, (KB + 3) // 4), dtype=np.uint32)
    for kb in range(KB):
        packed[0, kb // 4] |= np.uint32(kb) << np.uint32(8 * (kb % 4))
    got = oracle.unpack_ue8m0(packed, KB)[0]
    want = np.ldexp(np.float64(1.0), np.arange(KB) - 127).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    bits = got.view(np.uint32)
    assert bits[0] == 0x00400000
    assert np.array_equal(bits[1:], np.arange(1, KB, dtype=np.uint32) << np.uint32(23))


@pytest.mark.parametrize("KB", [1, 3, 4, 5, 56, 145])
def test_ue8m0_unpack_layout(KB):
    # byte j of word w is K-block 4w + j; the padding bytes of a row's last word are
    # ignored (filled with 255 here, which is not a scale)
    rng = np.random.default_rng(KB)
    rows = 3
    e = rng.integers(-20, 21, size=(rows, KB))
    words = (KB + 3) // 4
    b = np.full((rows, words * 4), 255, dtype=np.uint8)
    b[:, :KB] = (e + 127).astype(np.uint8)
    packed = b.view("<u4").reshape(rows, words)
    got = oracle.unpack_ue8m0(packed, KB)
    assert np.array_equal(got, np.ldexp(1.0, e).astype(np.float32))


def test_ue8m0_gemm_equals_fp32_scale_gemm():
    # the packed form only re-encodes power-of-two scales: the oracle's product is the
    # same bit for bit
    rng = np.random.default_rng(5)
    M, N, K = 5, 144, 640
    KB = K // 128
    A = rng.integers(0, 0x7F, size=(M, K), dtype=np.uint8)
    B = rng.integers(0, 0x7F, size=(N, K), dtype=np.uint8)
    e = rng.integers(-8, 9, size=(M, KB))
    sfA = np.ldexp(1.0, e).astype(np.float32)
    sfB = np.ldexp(1.0, rng.integers(-3, 4, size=((N + 127) // 128, KB))).astype(np.float32)
    b = np.zeros((M, 8), dtype=np.uint8)
    b[:, :KB] = e + 127
    packed = b.view("<u4").reshape(M, 2)
    r1 = oracle.gemm_nt(A, B, sfA, sfB)
    r2 = oracle.gemm_nt(A, B, oracle.unpack_ue8m0(packed, KB), sfB)
    assert np.array_equal(r1.view(np.uint64), r2.view(np.uint64))


# ------------------------------------------------------------------ SwiGLU


def _gu(g, u):
    g, u = np.atleast_2d(np.asarray(g, np.float64)), np.atleast_2d(np.asarray(u, np.float64))
    return np.concatenate([g, u], axis=-1)


def test_swiglu_closed_forms():
    # silu(0) = 0; silu(x) -> x for large x, -> 0 for very negative x; h scales with up
    h = oracle.swiglu(_gu([0.0, 40.0, -800.0, 1.0], [5.0, 1.0, 3.0, 2.0]))[0]
    assert h[0] == 0.0
    assert h[1] == 40.0  # exp(-40) < 2^-57: 40 / (1 + tiny) rounds to 40
    assert h[2] == 0.0 or abs(h[2]) < 1e-300
    # 1 / (1 + e^-1) is the logistic value at 1
    assert abs(h[3] - 2.0 / (1.0 + math.e ** -1)) <= 4e-16


def test_swiglu_identities():
    rng = np.random.default_rng(3)
    g = rng.normal(0, 6, 4096)
    one = np.ones_like(g)
    hp = oracle.swiglu(_gu(g, one))[0]
    hm = oracle.swiglu(_gu(-g, one))[0]
    # silu(x) - silu(-x) = x, since sigmoid(x) + sigmoid(-x) = 1
    assert np.allclose(hp - hm, g, rtol=0, atol=1e-13 * (1 + np.abs(g)))
    # other closed forms, through other library routines: x/2 (1 + tanh(x/2)) where it
    # does not cancel (x >= -1), x e^x / (1 + e^x) below
    t = np.array([x / 2 * (1 + math.tanh(x / 2)) if x >= -1 else
                  x * math.exp(x) / (1 + math.exp(x)) for x in g])
    assert np.allclose(hp, t, rtol=1e-14, atol=1e-300)
    # linear in up, exactly for powers of two
    u = rng.normal(size=g.size)
    h1 = oracle.swiglu(_gu(g, u))[0]
    h2 = oracle.swiglu(_gu(g, 4 * u))[0]
    assert np.array_equal(h2, 4 * h1)


def test_swiglu_layout_halves():
    # gate is the first half of each row, up the second; rows are independent
    gu = np.array([[1.0, 2.0, 10.0, 20.0], [3.0, 0.0, 1.0, 7.0]])
    h = oracle.swiglu(gu)
    assert h.shape == (2, 2)
    assert h[0, 0] == 1.0 / (1.0 + math.exp(-1.0)) * 10.0
    assert h[1, 1] == 0.0
