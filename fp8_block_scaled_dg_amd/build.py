"""Builds libdg.so (the HIP library) in-tree for gfx950 with hipcc."""
from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB_PATH = os.path.join(PKG, "libdg.so")
SOURCES = [os.path.join(CSRC, "dg_api.hip")]
DEPS = SOURCES + [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".hpp")] + [
    os.path.join(ROOT, "include", "dg.h")]
# measurement companion (streaming-read calibration kernel), loaded by the benchmark only
PROBE_LIB_PATH = os.path.join(PKG, "libdg_probe.so")
PROBE_SOURCES = [os.path.join(CSRC, "hbm_probe.hip")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-shared", "-fPIC",
    # no packed-fp32 VALU instructions (v_pk_*_f32) in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in ordinary VGPRs: the per-K-block promotion reads every partial
    # with VALU FMAs, which cannot take AGPR operands
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Wall", "-Wno-unused-function",
]


def source_hash() -> str:
    """Hash of the sources libdg.so is built from (every csrc file and dg.h): compiled
    into the library as its build id, and compared with the sources by the binding."""
    h = hashlib.sha256()
    for path in sorted(DEPS):
        with open(path, "rb") as f:
            h.update(os.path.basename(path).encode() + f.read())
    return h.hexdigest()[:16]


def command(out: str = LIB_PATH, extra: list[str] | None = None) -> list[str]:
    return ["hipcc", *HIPCC_FLAGS, f'-DDG_BUILD_ID="{source_hash()}"', *(extra or []), "-o", out,
            *SOURCES]


def _hipcc(cmd: list[str], what: str, verbose: bool) -> None:
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed building {what}")
    if verbose and msgs:
        sys.stderr.write("\n".join(msgs) + "\n")


def build(verbose: bool = False) -> str:
    _hipcc(command(), "libdg.so", verbose)
    _hipcc(["hipcc", *HIPCC_FLAGS, "-o", PROBE_LIB_PATH, *PROBE_SOURCES], "libdg_probe.so", verbose)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
