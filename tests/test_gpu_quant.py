"""GPU parity of the per-token 1x128 activation quantizer (dg_quantize_fp8_1x128)
against the oracle's block quantizer: the rule leaves no freedom (the scale is an
exact function of the block's largest magnitude, each code the nearest e4m3fn value
with ties to even), so codes and scale bits must match byte for byte.

Inputs: seeded N(0,1) rows (fp32 and bf16), blocks scaled over the whole fp32 /
bf16 exponent range, every e4m3fn rounding midpoint and its neighbours, zero and
negative-zero blocks, the 448 * 2^e scale boundary, fp32 subnormals (down to blocks
whose scale underflows to 0), ragged block counts, and the full 4096 x 18432 bf16
activation shape on sampled rows. Outputs sit between seeded guard bands that must
stay intact.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

GUARD = 4096


class GuardedBytes:
    """n output bytes inside a buffer with GUARD seeded random bytes either side."""

    def __init__(self, n: int, seed: int):
        rng = np.random.default_rng(seed)
        self.host = rng.integers(0, 256, size=n + 2 * GUARD, dtype=np.uint8)
        self.buf = torch.from_numpy(self.host.copy()).to("cuda")
        self.n = n

    def view(self, dtype, shape):
        return self.buf[GUARD:GUARD + self.n].view(dtype).view(*shape)

    def result(self) -> np.ndarray:
        return self.buf[GUARD:GUARD + self.n].cpu().numpy()

    def guards_intact(self) -> bool:
        now = self.buf.cpu().numpy()
        return (np.array_equal(now[:GUARD], self.host[:GUARD])
                and np.array_equal(now[GUARD + self.n:], self.host[GUARD + self.n:]))


def run_quant(x: torch.Tensor, seed: int = 5):
    import fp8_block_scaled_dg_amd as dg
    M, K = x.shape
    codes = GuardedBytes(M * K, seed)
    sf = GuardedBytes(M * (K // 128) * 4, seed + 1)
    gu.announce(f"quantize {x.dtype} M={M} K={K}")
    dg.quantize_fp8_1x128(x, codes.view(torch.float8_e4m3fn, (M, K)),
                          sf.view(torch.float32, (M, K // 128)))
    torch.cuda.synchronize()
    assert codes.guards_intact() and sf.guards_intact(), "write outside the outputs"
    return codes.result().reshape(M, K), sf.result().view(np.float32).reshape(M, K // 128)


def check_exact(x32: np.ndarray, codes: np.ndarray, sf: np.ndarray, what: str):
    rc, rs = oracle.quantize_blocks(x32, 1, 128)
    bad_s = np.nonzero(rs.view(np.uint32) != sf.view(np.uint32))
    assert bad_s[0].size == 0, (f"{what}: {bad_s[0].size} scales differ, first at {bad_s[0][0]},"
                                f"{bad_s[1][0]}: {sf[bad_s][0]!r} vs {rs[bad_s][0]!r}")
    bad = np.nonzero(codes != rc)
    assert bad[0].size == 0, (f"{what}: {bad[0].size} codes differ, first at ({bad[0][0]},"
                              f"{bad[1][0]}): x={x32[bad][0]!r} gpu={codes[bad][0]:#04x} "
                              f"oracle={rc[bad][0]:#04x}")


def as_bf16_exact(x32: np.ndarray):
    """(bf16 device tensor, its values as fp32 numpy): the bf16 rounding is input
    preparation; the oracle sees exactly the values the kernel reads."""
    t = torch.from_numpy(x32).to(torch.bfloat16)
    return t.to("cuda"), t.to(torch.float32).numpy()


@pytest.mark.parametrize("M,K", [(1, 128), (3, 384), (257, 1152), (64, 7168)])
def test_gaussian_fp32_and_bf16(M, K):
    x = synth.normal_rows(77000 + M, M, K)
    codes, sf = run_quant(torch.from_numpy(x).to("cuda"))
    check_exact(x, codes, sf, f"fp32 {M}x{K}")
    xb, xb32 = as_bf16_exact(x)
    codes, sf = run_quant(xb)
    check_exact(xb32, codes, sf, f"bf16 {M}x{K}")


def test_exponent_range():
    # every block scaled by its own power of two, across the representable range
    rng = np.random.default_rng(11)
    M, K = 96, 1024
    x = synth.normal_rows(77100, M, K).astype(np.float64)
    k32 = rng.integers(-140, 121, size=(M, K // 128))
    x32 = np.ldexp(x, np.repeat(k32, 128, axis=1)).astype(np.float32)
    codes, sf = run_quant(torch.from_numpy(x32).to("cuda"))
    check_exact(x32, codes, sf, "fp32 exponent range")
    k16 = rng.integers(-120, 121, size=(M, K // 128))
    xb, xb32 = as_bf16_exact(np.ldexp(x, np.repeat(k16, 128, axis=1)).astype(np.float32))
    codes, sf = run_quant(xb)
    check_exact(xb32, codes, sf, "bf16 exponent range")


def test_every_rounding_midpoint():
    vals = oracle.e4m3fn_values()[:127]  # the finite non-negative values, in order
    ys = np.concatenate([vals, (vals[:-1] + vals[1:]) / 2]).astype(np.float32).astype(np.float64)
    ys = np.concatenate([ys, np.nextafter(ys, np.inf), np.nextafter(ys, -np.inf)])
    ys = ys[(ys >= 0) & (ys <= 448)]
    ys = np.concatenate([ys, -ys]).astype(np.float32)
    n = (ys.size // 127) * 127
    blocks = ys[:n].reshape(-1, 127)
    # first value 448 pins the block's scale to 2^j, j set per block below
    x = np.concatenate([np.full((blocks.shape[0], 1), 448.0, np.float32), blocks], axis=1)
    rows = []
    for j in (0, -7, 5, -60, 40):
        rows.append(np.ldexp(x.astype(np.float64), j).astype(np.float32))
    x32 = np.concatenate(rows).reshape(-1, 128)
    codes, sf = run_quant(torch.from_numpy(x32).to("cuda"))
    check_exact(x32, codes, sf, "midpoints")


def test_special_blocks():
    K = 128
    blocks = []
    blocks.append(np.zeros(K, np.float32))                                   # amax 0 -> scale 1
    blocks.append(np.full(K, -0.0, np.float32))                              # sign of zero
    b = np.linspace(-1, 1, K).astype(np.float32); b[7] = 448.0               # scale exactly 1
    blocks.append(b)
    b = b.copy(); b[7] = np.nextafter(np.float32(448), np.float32(np.inf))   # just above -> 2
    blocks.append(b)
    for a in (1.75, np.nextafter(np.float32(1.75), np.float32(2)), 0.875, 1.0, 3.0e38):
        b = np.linspace(-0.5, 0.5, K).astype(np.float32) * np.float32(min(a, 1.0))
        b[100] = np.float32(a)
        blocks.append(b)
    one = np.zeros(K, np.float32); one[50] = -3.0                            # single nonzero
    blocks.append(one)
    tiny = np.full(K, np.float32(1e-30)); tiny[3] = np.float32(-1e-33)       # values -> -0 code
    tiny[4] = np.float32(1e-30) * np.float32(2.0 ** -12)
    blocks.append(tiny)
    # fp32 subnormals: amax 2^-149 (scale 2^-157 underflows to 0), 2^-130, and mixes
    for amax_exp in (-149, -145, -141, -140, -135, -130, -127, -126):
        b = np.zeros(K, np.float32)
        b[:] = np.ldexp(np.linspace(-1, 1, K), amax_exp).astype(np.float32)
        b[9] = np.float32(np.ldexp(1.0, amax_exp))
        blocks.append(b)
    x32 = np.stack(blocks).astype(np.float32)
    x32 = np.concatenate([x32, -x32[::-1]])                                   # both signs
    codes, sf = run_quant(torch.from_numpy(x32.reshape(-1, 2 * K)).to("cuda"))
    check_exact(x32.reshape(-1, 2 * K), codes, sf, "special blocks")


def test_zero_rows_is_a_noop():
    import fp8_block_scaled_dg_amd as dg
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device="cuda")
    codes, sf = dg.quantize_fp8_1x128(x)
    torch.cuda.synchronize()
    assert codes.shape == (0, 256) and sf.shape == (0, 2)


def test_activation_workload_sampled():
    # the prefill GEMM's A operand: bf16 [4096][18432], the bench's quantizer workload;
    # its 589,824 blocks run through the kernel's grid-stride loop
    M, K = 4096, 18432
    x = synth.normal_rows(3001, M, K)
    xb = torch.from_numpy(x).to(torch.bfloat16)
    codes, sf = run_quant(xb.to("cuda"))
    rng = np.random.default_rng(12)
    rows = np.unique(np.concatenate([[0, 1, 2047, 2048, M - 1], rng.integers(0, M, 59)]))
    xs = xb[rows].to(torch.float32).numpy()
    check_exact(xs, codes[rows], sf[rows], "activation workload rows")
