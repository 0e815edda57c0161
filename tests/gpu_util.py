"""Helpers for GPU tests: host<->device transfer, sentinel-filled outputs with guard
bands, calls through the binding. Imported by GPU tests only."""
from __future__ import annotations

import sys

import numpy as np
import torch

GUARD = 64 * 1024  # bytes of guard band on each side of an output buffer


def dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x)).to("cuda")
    if dtype is not None and dtype == torch.float8_e4m3fn:
        t = t.view(torch.float8_e4m3fn)
    return t


def codes(x: np.ndarray) -> torch.Tensor:
    return dev(x.astype(np.uint8)).view(torch.float8_e4m3fn)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


class Guarded:
    """A bf16 output of `shape` inside a buffer with GUARD bytes either side, all
    filled with seeded random bytes (NaN payloads included)."""

    def __init__(self, shape, seed: int):
        n = int(np.prod(shape))
        g = GUARD // 2
        rng = np.random.default_rng(seed)
        self.host = rng.integers(0, 1 << 16, size=n + 2 * g, dtype=np.uint16)
        self.buf = torch.from_numpy(self.host.view(np.int16).copy()).to("cuda")
        self.out = self.buf[g:g + n].view(torch.bfloat16).view(*shape)
        self.g, self.n, self.shape = g, n, tuple(shape)

    def result(self) -> np.ndarray:
        return bits(self.out).reshape(self.shape)

    def initial(self) -> np.ndarray:
        return self.host[self.g:self.g + self.n].reshape(self.shape)

    def guards_intact(self) -> bool:
        now = self.buf.cpu().numpy().view(np.uint16)
        return (np.array_equal(now[:self.g], self.host[:self.g])
                and np.array_equal(now[self.g + self.n:], self.host[self.g + self.n:]))


def announce(msg: str) -> None:
    """Name the case on stdout before a GPU step, flushed, so a fault is attributable."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()
