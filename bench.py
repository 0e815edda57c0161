#!/usr/bin/env python3
"""Benchmark of the FP8 block-scaled GEMM library on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode]

A step is one pass of every GEMM in the workload over one batch of synthetic
inputs already resident in HBM. The default workload is the pair of memory-bound
decode shapes at M = 64 (64x2112x7168 and 64x32768x512, the shapes of the launch
article's benchmark table, section 2.1); the metric is achieved algorithmic HBM
throughput in GB/s. Other workloads (--workload prefill | moe_cont | moe_mask |
small) report TFLOPS against the dense FP8 MFMA peak.

Timing: W untimed warmup steps (more if they take under --warmup-seconds, so that
the clocks have ramped up from idle; the JSON reports the count run), then exactly
K steps between two synchronisations.
The K launches of each GEMM run back to back between a pair of HIP events
(torch.cuda.Event, on the stream the kernels are launched on), which gives each
kernel's average launch duration. Input and output buffers rotate over enough
copies that their total exceeds 512 MB, so neither L2 nor the 256 MB MALL holds
the previous step's operands.

Prints one JSON line. The roofline object covers the kernel with the largest total
time: algorithmic bytes (or FLOPs) per launch / its average event-timed duration
against MI355X's published peak (HBM 8 TB/s; dense FP8 MFMA 5.0 PFLOP/s).
cpu_baseline is the CPU oracle timed on the host's cores over the whole step
(reported as a baseline only), and that same leg compares the GPU outputs of the
last timed step with the oracle.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0
MAX_COPIES = 64  # rotation sets per GEMM: enough to defeat L2 and MALL, few enough to set up
PEAK_CLOCK_GHZ = 2.4  # the clock the published FP8 peak is quoted at
DECODE_BYTES = {"dec2112": 15886048, "dec32768": 21009408}
METRIC = "FP8 block-scaled GEMM TFLOPS (%MFMA peak) and GB/s at M=64 (%HBM), 1 MI355X"

WORKLOADS = {
    "decode": ["dec2112", "dec32768"],
    "prefill": ["prefill"],
    "moe_cont": ["moe_cont"],
    "moe_mask": ["moe_mask"],
    "small": ["small"],
    "quant": ["quant_act"],
    "moe_swiglu": ["moe_cont_swiglu"],
}
DESCRIPTIONS = {
    "decode": "dense NT decode, M=64: 64x2112x7168 + 64x32768x512",
    "prefill": "dense NT prefill 4096x7168x18432",
    "moe_cont": "MoE grouped contiguous, 32 experts, N=4096, K=7168, 8192 Zipf-routed tokens",
    "moe_mask": "MoE grouped masked, 32 experts x 256 rows, N=7168, K=2048",
    "small": "dense NT 128x256x512",
    "quant": "per-token 1x128 FP8 quantization of bf16 activations [4096][18432] "
             "(the prefill GEMM's A operand and sfA)",
}
DESCRIPTIONS["moe_swiglu"] = ("MoE grouped contiguous Linear1 with the fused SwiGLU + 1x128 "
                              "requantization epilogue: 32 experts, B = [gate; up] with I = 2048, "
                              "K=7168, 8192 Zipf-routed tokens")
QUANT_SHAPES = {"quant_act": (4096, 18432, 3001)}  # M, K, seed of the N(0,1) rows


class Gemm:
    """One GEMM of the workload: host inputs, device copies, algorithmic work."""

    def __init__(self, name, w, sfa_layout: str = "f32", layout: str = "nt"):
        import numpy as np
        self.name, self.w = name, w
        self.layout = layout
        self.kind = type(w).__name__.lower()
        if self.kind == "dense":
            M, N, K = w.shape
            Mv, Ga, G = M, 1, 1
            meta = 0
        elif self.kind == "contiguous":
            M, N, K, G = w.shape
            Mv = int(w.counts.sum())
            Ga = int((w.counts > 0).sum())
            meta = 4 * M
        else:
            G, M, N, K = w.shape
            Mv = int(np.clip(w.masked_m, 0, M).sum())
            Ga = int((np.clip(w.masked_m, 0, M) > 0).sum())
            meta = 4 * G
        KB, NB = K // 128, (N + 127) // 128
        sfa_row = 4 * ((KB + 3) // 4) if sfa_layout == "ue8m0" else 4 * KB  # bytes per row
        self.flops = 2.0 * Mv * N * K
        self.bytes = (Mv * K + Ga * N * K + Mv * sfa_row + 4 * Ga * NB * KB + 2 * Mv * N + meta)
        self.shape = dict(M=M, N=N, K=K, G=G, valid_rows=Mv, active_experts=Ga)
        self.footprint = (w.A.nbytes + w.B.nbytes + w.sfA.nbytes + w.sfB.nbytes
                          + (M * N * 2 if self.kind != "masked" else G * M * N * 2))

    def upload(self, copies: int, sfa_layout: str = "f32"):
        import numpy as np
        import torch
        import synth
        dev = torch.device("cuda:0")

        def t(x):
            return torch.from_numpy(x).to(dev)

        sfa = synth.pack_ue8m0(self.w.sfA) if sfa_layout == "ue8m0" else self.w.sfA
        a_host, b_host = self.w.A, self.w.B
        if self.kind == "dense" and self.layout[0] == "t":
            a_host = np.ascontiguousarray(a_host.T)  # A stored [K][M]
        if self.kind == "dense" and self.layout[1] == "n":
            b_host = np.ascontiguousarray(b_host.T)  # B stored [K][N]
        base = dict(A=t(a_host).view(torch.float8_e4m3fn), B=t(b_host).view(torch.float8_e4m3fn),
                    sfA=t(sfa), sfB=t(self.w.sfB))
        if self.kind == "contiguous":
            base["idx"] = t(self.w.m_indices)
            cshape = (self.w.A.shape[0], self.w.B.shape[1])
        elif self.kind == "masked":
            base["idx"] = t(self.w.masked_m)
            cshape = (self.w.A.shape[0], self.w.A.shape[1], self.w.B.shape[1])
        else:
            cshape = (self.w.A.shape[0], self.w.B.shape[0])
        self.sets = []
        for i in range(copies):
            s = {k: (v if i == 0 else v.clone()) for k, v in base.items()}
            s["C"] = torch.zeros(cshape, dtype=torch.bfloat16, device=dev)
            self.sets.append(s)

    def launch(self, i: int):
        import fp8_block_scaled_dg_amd as dg
        s = self.sets[i % len(self.sets)]
        if self.kind == "dense":
            getattr(dg, "fp8_gemm_" + self.layout)(s["A"], s["B"], s["C"], s["sfA"], s["sfB"])
        elif self.kind == "contiguous":
            dg.m_grouped_fp8_gemm_nt_contiguous(s["A"], s["B"], s["C"], s["sfA"], s["sfB"],
                                                s["idx"])
        else:
            dg.m_grouped_fp8_gemm_nt_masked(s["A"], s["B"], s["C"], s["sfA"], s["sfB"], s["idx"],
                                            int(self.w.masked_m.mean()))


class SwigluGemm(Gemm):
    """The contiguous MoE workload as Linear1 of a layer (B = [gate; up], I = N/2) with
    the fused epilogue: outputs e4m3fn codes [M_total][I] and fp32 scales [M_total][I/128]
    instead of bf16 C."""

    def __init__(self, name, w, sfa_layout: str = "f32"):
        super().__init__(name, w)
        M, N, K = self.shape["M"], self.shape["N"], self.shape["K"]
        Mv = self.shape["valid_rows"]
        self.I = N // 2
        # bf16 C replaced by codes (1 byte) and scales (4 bytes per 128 values)
        self.bytes += -2 * Mv * N + Mv * self.I + 4 * Mv * (self.I // 128)
        self.footprint += -M * N * 2 + M * self.I * 5 // 4

    def upload(self, copies: int, sfa_layout: str = "f32"):
        import torch
        super().upload(copies, "f32")
        M = self.shape["M"]
        for st in self.sets:
            del st["C"]
            st["codes"] = torch.empty((M, self.I), dtype=torch.float8_e4m3fn, device="cuda:0")
            st["sf"] = torch.empty((M, self.I // 128), dtype=torch.float32, device="cuda:0")

    def launch(self, i: int):
        import fp8_block_scaled_dg_amd as dg
        s = self.sets[i % len(self.sets)]
        dg.m_grouped_fp8_gemm_nt_contiguous_swiglu(s["A"], s["B"], s["sfA"], s["sfB"], s["idx"],
                                                   s["codes"], s["sf"])


def swiglu_oracle_leg(g, last_set: int, budget_macs: float = 4e9):
    """Oracle chain (grouped products, fp64 SwiGLU, quantizer) on seeded whole rows,
    timed and scaled to every produced row; the last timed step's codes and scales at
    those rows are compared with it (the kernel forms h in fp32, so a code may differ
    where h sits within its error of a rounding boundary)."""
    import numpy as np
    import torch
    import oracle
    w, I = g.w, g.I
    N2, K = g.shape["N"], g.shape["K"]
    rows = np.nonzero(w.m_indices >= 0)[0]
    n_rows = rows.size
    take = int(min(n_rows, max(1, budget_macs // (N2 * K))))
    rows = np.sort(np.random.default_rng(12345).choice(rows, take, replace=False))
    ri = np.repeat(rows, N2).astype(np.int64)
    ni = np.tile(np.arange(N2, dtype=np.int64), rows.size)
    reps, dt = 0, 0.0
    while reps == 0 or dt < 1.0:
        t0 = time.perf_counter()
        gu = oracle.grouped_contiguous_at(w.A, w.B, w.sfA, w.sfB, w.m_indices, ri, ni)
        h = oracle.swiglu(gu.reshape(rows.size, N2))
        rc, rs = oracle.quantize_blocks(h.astype(np.float32), 1, 128)
        dt += time.perf_counter() - t0
        reps += 1
    dt /= reps
    st = g.sets[last_set % len(g.sets)]
    codes = st["codes"].view(torch.uint8).cpu().numpy()[rows]
    sf = st["sf"].cpu().numpy()[rows]
    check = dict(n=int(rc.size), code_match=float((codes == rc).mean()),
                 scale_match=float((sf == rs).mean()))
    sample = f"{g.name}: {rows.size} of {n_rows} rows x {N2} gate/up columns, {dt:.3f} s (mean of {reps})"
    return dt * n_rows / rows.size, sample, {g.name: check}


class Quant:
    """The per-token 1x128 activation quantizer over bf16 activations [M][K]: one read
    of x (2 bytes a value), one write of the codes (1 byte) and of the scales (4 bytes
    per 128 values)."""

    def __init__(self, name, M, K, seed):
        import torch
        import synth
        self.name, self.kind = name, "quant"
        # input preparation: seeded N(0,1) values rounded to bf16
        self.x_host = torch.from_numpy(synth.normal_rows(seed, M, K)).to(torch.bfloat16)
        self.flops = 0.0
        self.bytes = M * K * 2 + M * K + M * (K // 128) * 4
        self.shape = dict(M=M, K=K, x_dtype="bf16")
        self.footprint = self.bytes

    def upload(self, copies: int, sfa_layout: str = "f32"):
        import torch
        dev = torch.device("cuda:0")
        M, K = self.shape["M"], self.shape["K"]
        x = self.x_host.to(dev)
        self.sets = [dict(x=x if i == 0 else x.clone(),
                          codes=torch.empty((M, K), dtype=torch.float8_e4m3fn, device=dev),
                          sf=torch.empty((M, K // 128), dtype=torch.float32, device=dev))
                     for i in range(copies)]

    def launch(self, i: int):
        import fp8_block_scaled_dg_amd as dg
        s = self.sets[i % len(self.sets)]
        dg.quantize_fp8_1x128(s["x"], s["codes"], s["sf"])


def quant_oracle_leg(q, last_set: int, budget_values: float = 8e6):
    """The oracle's block quantizer on a seeded sample of whole rows, timed and scaled
    to the whole tensor; the last timed step's codes and scales at those rows must
    equal it byte for byte."""
    import numpy as np
    import torch
    import oracle
    M, K = q.shape["M"], q.shape["K"]
    take = int(min(M, max(1, budget_values // K)))
    rows = np.sort(np.random.default_rng(12345).choice(M, take, replace=False))
    x = q.x_host[torch.from_numpy(rows)].to(torch.float32).numpy()
    reps, dt = 0, 0.0
    while reps == 0 or dt < 1.0:
        t0 = time.perf_counter()
        rc, rs = oracle.quantize_blocks(x, 1, 128)
        dt += time.perf_counter() - t0
        reps += 1
    dt /= reps
    s = q.sets[last_set % len(q.sets)]
    codes = s["codes"].view(torch.uint8).cpu().numpy()[rows]
    sf = s["sf"].cpu().numpy()[rows]
    check = dict(n=int(rc.size), code_mismatch=int((codes != rc).sum()),
                 scale_mismatch=int((sf.view(np.uint32) != rs.view(np.uint32)).sum()))
    sample = f"{q.name}: {take} of {M} rows x {K} values, {dt:.3f} s (mean of {reps})"
    return dt * M / take, sample, {q.name: check}


def oracle_leg(gemms, last_set: int, sfa_layout: str = "f32", budget_macs: float = 4e9):
    """CPU baseline: the oracle over the step's produced outputs -- every output when a
    GEMM is at most budget_macs multiply-adds, else a seeded sample of whole rows --
    timed on the host cores and scaled to the whole step; and the comparison of the
    last timed step's GPU outputs with it at the same positions."""
    import numpy as np
    import torch
    import oracle
    from tests.parity import report

    per_step, checks, samples = 0.0, {}, []
    import synth
    for g in gemms:
        w = g.w
        N, K = g.shape["N"], g.shape["K"]
        # the oracle reads the scales in the layout the GPU was given
        sfA = (oracle.unpack_ue8m0(synth.pack_ue8m0(w.sfA), K // 128) if sfa_layout == "ue8m0"
               else w.sfA)
        if g.kind == "dense":
            rows = np.arange(g.shape["M"])
        elif g.kind == "contiguous":
            rows = np.nonzero(w.m_indices >= 0)[0]
        else:
            M_max = g.shape["M"]
            prod = np.arange(M_max)[None, :] < np.clip(w.masked_m, 0, M_max)[:, None]
            rows = np.nonzero(prod.ravel())[0]  # flat e * M_max + m
        n_rows = rows.size
        take = int(min(n_rows, max(1, budget_macs // (N * K))))
        if take < n_rows:
            rows = np.sort(np.random.default_rng(12345).choice(rows, take, replace=False))
        ri = np.repeat(rows, N).astype(np.int64)
        ni = np.tile(np.arange(N, dtype=np.int64), rows.size)
        reps, dt = 0, 0.0
        while reps == 0 or dt < 1.0:  # repeat short samples for a stable time
            t0 = time.perf_counter()
            if g.kind == "dense":
                r = oracle.gemm_nt_at(w.A, w.B, sfA, w.sfB, ri, ni)
            elif g.kind == "contiguous":
                r = oracle.grouped_contiguous_at(w.A, w.B, sfA, w.sfB, w.m_indices, ri, ni)
            else:
                M_max = g.shape["M"]
                r = oracle.grouped_masked_at(w.A, w.B, sfA, w.sfB, w.masked_m, ri // M_max,
                                             ri % M_max, ni)
            dt += time.perf_counter() - t0
            reps += 1
        dt /= reps
        per_step += dt * n_rows / rows.size
        samples.append(f"{g.name}: {rows.size} of {n_rows} rows x {N} cols, {dt:.3f} s "
                       f"(mean of {reps})")
        C = g.sets[last_set % len(g.sets)]["C"].view(torch.int16).cpu().numpy().view(np.uint16)
        gpu = C.reshape(-1, N)[ri, ni]
        rep = report(gpu, r)
        checks[g.name] = {k: rep[k] for k in ("n", "max_excess_rel", "bitwise_match", "n_fail",
                                               "nan")}
    return per_step, "; ".join(samples), checks


class ClockSampler:
    """Samples the GPU's current shader (gfx) clock through amdsmi in a background
    thread while a timed region runs; mean() is the average over the samples (MHz),
    or None where amdsmi reports nothing."""

    def __init__(self, period_s: float = 0.002):
        import threading
        self.period, self.samples, self._stop = period_s, [], threading.Event()
        self._thread, self.handle = None, None
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            self.amdsmi, self.handle = amdsmi, (handles[0] if handles else None)
        except Exception:  # no amdsmi, or no access: the clock stays unreported
            self.handle = None

    def _read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        xs = [x for x in (m.get("current_gfxclks") or []) if isinstance(x, (int, float)) and x > 0]
        if xs:
            return sum(xs) / len(xs)
        x = m.get("current_gfxclk")
        return float(x) if isinstance(x, (int, float)) and x > 0 else None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except Exception:
                return
            if v:
                self.samples.append(v)
            self._stop.wait(self.period)

    def __enter__(self):
        import threading
        if self.handle is not None:
            self._thread = threading.Thread(target=self._run, daemon=True)
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self._thread:
            self._thread.join()

    def mean(self):
        return sum(self.samples) / len(self.samples) if self.samples else None


def timed_launches(launch, K: int, start: int, graph: bool, sampler=None):
    """Average duration (ms) of K back-to-back launches launch(start), ..., launch(start
    + K - 1), between two HIP events on the stream the launches run on. graph: the K
    launches are first captured into one HIP graph on a side stream (after a warm call
    there, so that the library's per-stream buffers exist) and the replay is timed:
    the GPU then runs them back to back without host launch gaps."""
    import torch
    s = torch.cuda.Stream() if graph else torch.cuda.current_stream()
    g = None
    if graph:
        with torch.cuda.stream(s):
            launch(start)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(K):
                launch(start + i)
        torch.cuda.synchronize()
        with torch.cuda.stream(s):  # one untimed replay
            g.replay()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ctx = sampler if sampler is not None else _Null()
    with torch.cuda.stream(s), ctx:
        e0.record(s)
        if graph:
            g.replay()
        else:
            for i in range(K):
                launch(start + i)
        e1.record(s)
        e1.synchronize()
    return e0.elapsed_time(e1) / K


class _Null:
    def __enter__(self):
        return self

    def __exit__(self, *exc):
        return False


def hbm_ceiling(nbytes_list, rotate_bytes: int, reps: int = 50):
    """The streaming-read probe (libdg_probe.so) on each byte count, rotated over
    rotate_bytes of buffers, graph-timed: the best over grid sizes and load kinds of
    the average per-launch time, and the empty-kernel time."""
    import ctypes
    import torch
    from fp8_block_scaled_dg_amd import build as dgb
    lib = ctypes.CDLL(dgb.PROBE_LIB_PATH)
    lib.dg_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                         ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
    lib.dg_probe_empty.argtypes = [ctypes.c_void_p]
    sink = torch.empty(8192, dtype=torch.int32, device="cuda:0")
    out = {}
    for nb in nbytes_list:
        nb16 = nb // 16 * 16
        copies = max(1, min(64, -(-rotate_bytes // nb16)))
        bufs = [torch.empty(nb16, dtype=torch.uint8, device="cuda:0").fill_(i % 251)
                for i in range(copies)]
        best = None
        for blocks in (256, 512, 1024, 2048):
            for nt in (0, 1):
                def launch(i, blocks=blocks, nt=nt):
                    st = torch.cuda.current_stream().cuda_stream
                    rc = lib.dg_probe_stream_read(bufs[i % copies].data_ptr(), nb16,
                                                  sink.data_ptr(), blocks, nt, st)
                    assert rc == 0, rc
                ms = timed_launches(launch, reps, 0, graph=True)
                if best is None or ms < best[0]:
                    best = (ms, blocks, nt)
        out[str(nb)] = dict(bytes=nb16, us=best[0] * 1e3, gbs=nb16 / (best[0] * 1e-3) / 1e9,
                            blocks=best[1], nontemporal=bool(best[2]))
        del bufs

    def empty(i):
        assert lib.dg_probe_empty(torch.cuda.current_stream().cuda_stream) == 0
    out["empty_kernel_us"] = timed_launches(empty, reps, 0, graph=True) * 1e3
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep running untimed warmup steps past --warmup until this much "
                         "time has passed, so that the GPU clocks have left their idle state "
                         "(0: exactly --warmup steps, e.g. under a profiler)")
    ap.add_argument("--workload", default="decode",
                    choices=sorted(WORKLOADS) + ["hbm_ceiling", "vendor_prefill", "vendor_decode",
                                                 "overlap_probe"])
    ap.add_argument("--timing", choices=("graph", "eager"), default="graph",
                    help="graph: the K launches of each GEMM are captured into a HIP graph "
                         "and replayed (no host launch gaps); eager: launched from Python")
    ap.add_argument("--rotate-mb", type=int, default=512,
                    help="input/output sets rotate over this many MB (0: one set); at most "
                         f"{MAX_COPIES} copies")
    ap.add_argument("--no-prefill", action="store_true",
                    help="skip the compute-bound prefill leg of the default decode run")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the streaming-read ceiling of the default decode run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", choices=("nt", "nn", "tn", "tt"), default="nt",
                    help="memory layout of the dense GEMMs' operands (A [K][M] for t, "
                         "B [K][N] for n); the timed call includes the transposition")
    ap.add_argument("--sfa", choices=("f32", "ue8m0"), default="f32",
                    help="layout of the A scales: fp32 values, or packed UE8M0 exponent bytes")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 256 MiB device copy (to calibrate HBM counters)")
    ap.add_argument("--gemm", default=None,
                    help="run only this GEMM of the workload (for per-kernel counter runs)")
    ap.add_argument("--summarize", metavar="MANIFEST", default=None,
                    help="write profiles/ summaries from rocprofv3 outputs listed in MANIFEST "
                         "(JSON); runs on the host, no GPU needed")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize)
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: this library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE={world}). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    if args.copy_calibration:
        copy_calibration()
        return
    import synth
    import fp8_block_scaled_dg_amd as dg  # fails loudly if libdg.so is missing or stale

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    rotate = args.rotate_mb * 1024 * 1024
    if args.workload == "hbm_ceiling":
        ceil = hbm_ceiling([DECODE_BYTES["dec2112"], DECODE_BYTES["dec32768"]], rotate)
        print(json.dumps({"metric": "streaming-read GB/s at the decode GEMMs' byte counts",
                          "value": ceil[str(DECODE_BYTES["dec2112"])]["gbs"], "unit": "GB/s",
                          "n_gpus": 1, "higher_is_better": True, "data": "synthetic",
                          "config": {"workload": "plain streaming read (libdg_probe.so)"},
                          "hbm_ceiling": ceil}), flush=True)
        return
    if args.workload == "vendor_prefill":
        print(json.dumps(vendor_prefill(args.steps, rotate)), flush=True)
        return
    if args.workload == "vendor_decode":
        print(json.dumps(vendor_decode(args.steps, rotate)), flush=True)
        return
    if args.workload == "overlap_probe":
        print(json.dumps({"metric": "ns per iteration of the overlap probe (libdg_probe.so)",
                          "unit": "ns", "n_gpus": 1, "higher_is_better": False,
                          "data": "synthetic", "overlap": overlap_probe()}), flush=True)
        return
    names = WORKLOADS[args.workload]
    if args.gemm is not None:
        if args.gemm not in names:
            sys.exit(f"--gemm {args.gemm} is not part of workload {args.workload}: {names}")
        names = [args.gemm]
    gemms = [Quant(n, *QUANT_SHAPES[n]) if n in QUANT_SHAPES else
             SwigluGemm(n, synth.workload("moe_cont")) if n == "moe_cont_swiglu" else
             Gemm(n, synth.workload(n), args.sfa, args.layout)
             for n in names]
    step_footprint = sum(g.footprint for g in gemms)
    copies = max(1, min(MAX_COPIES, -(-rotate // step_footprint)))
    for g in gemms:
        g.upload(copies, args.sfa)
    torch.cuda.synchronize()

    warm = 0
    t0 = time.perf_counter()
    while warm < args.warmup or time.perf_counter() - t0 < args.warmup_seconds:
        chunk = max(1, args.warmup - warm) if warm < args.warmup else max(1, warm)
        for s in range(warm, warm + chunk):
            for g in gemms:
                g.launch(s)
        warm += chunk
        torch.cuda.synchronize()
    warmup_run = warm  # the number of untimed steps actually run

    # Timed region: the K steps' launches, grouped by GEMM (all K launches of one GEMM
    # back to back on rotating buffers, then the next GEMM), each group bracketed by
    # events on its launch stream: a group's elapsed time / K is that kernel's average
    # launch duration, and the sum over the groups is the time of one step. With graph
    # timing a group is one replayed HIP graph of its K launches; the eager figures
    # (launches from Python, host launch gaps included) are reported beside it.
    K = args.steps
    graph = args.timing == "graph"
    # eager first, so that under a kernel trace each GEMM's last K dispatches are the
    # timed ones of the reported figure
    eager_ms = [timed_launches(g.launch, K, warmup_run, False) for g in gemms] if graph else None
    wall0 = time.perf_counter()
    per_ms = [timed_launches(g.launch, K, warmup_run, graph) for g in gemms]
    wall = time.perf_counter() - wall0
    eager_ms = eager_ms or per_ms
    ms_per_step = sum(per_ms)
    last_set = warmup_run + K - 1

    kern = []
    for j, g in enumerate(gemms):
        ms = per_ms[j]
        kern.append(dict(name=g.name, shape=g.shape, avg_us=ms * 1e3,
                         eager_avg_us=eager_ms[j] * 1e3,
                         tflops=g.flops / (ms * 1e-3) / 1e12,
                         gbs=g.bytes / (ms * 1e-3) / 1e9,
                         alg_bytes=g.bytes, alg_flops=g.flops))
    step_bytes = sum(g.bytes for g in gemms)
    step_flops = sum(g.flops for g in gemms)
    memory_bound = args.workload in ("decode", "quant")
    if memory_bound:
        value, unit = step_bytes / (ms_per_step * 1e-3) / 1e9, "GB/s"
    else:
        value, unit = step_flops / (ms_per_step * 1e-3) / 1e12, "TFLOPS"

    dom = max(range(len(gemms)), key=lambda j: kern[j]["avg_us"])
    kd = kern[dom]
    t_mem = kd["alg_bytes"] / (HBM_PEAK_GBS * 1e9)
    t_mfma = kd["alg_flops"] / (FP8_PEAK_TFLOPS * 1e12)
    if memory_bound or t_mem > t_mfma:
        roof = dict(bound="hbm", achieved=kd["gbs"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=kd["gbs"] / HBM_PEAK_GBS)
    else:
        roof = dict(bound="mfma", achieved=kd["tflops"], peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=kd["tflops"] / FP8_PEAK_TFLOPS)
    roof["kernel"] = kd["name"]
    roof["traffic"] = measured_traffic(kd["name"], dg.BUILD_ID)

    line_extra = {}
    if args.workload == "decode" and not args.no_ceiling and args.gemm is None:
        ceil = hbm_ceiling([g.bytes for g in gemms], rotate)
        line_extra["hbm_ceiling"] = ceil
        c = ceil[str(kd["alg_bytes"])]
        roof["ceiling_gbs"] = c["gbs"]
        roof["frac_of_ceiling"] = kd["gbs"] / c["gbs"]
    if args.workload == "decode" and not args.no_prefill and args.gemm is None:
        line_extra.update(prefill_leg(max(K, 50), rotate, graph))
        line_extra["roofline_mfma"] = line_extra["prefill"].pop("roofline")

    cpu = None
    if not args.no_cpu_baseline:
        if args.workload == "quant":
            per_step, sample, checks = quant_oracle_leg(gemms[0], last_set)
        elif args.workload == "moe_swiglu":
            per_step, sample, checks = swiglu_oracle_leg(gemms[0], last_set)
        else:
            per_step, sample, checks = oracle_leg(gemms, last_set, args.sfa)
        import oracle
        cores = oracle.num_threads()
        cpu_value = (step_bytes / per_step / 1e9) if memory_bound else (step_flops / per_step / 1e12)
        cpu = dict(value=cpu_value, unit=unit, cores=cores, kind="oracle",
                   sample=sample + f"; scaled to the whole step: {per_step:.2f} s",
                   parity=checks)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": K,
        "warmup": warmup_run,
        "warmup_requested": args.warmup,
        "ms_per_step": ms_per_step,
        "eager_ms_per_step": sum(eager_ms),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32" if args.workload == "quant" else "fp8",
        "data": "synthetic",
        "config": ({"workload": DESCRIPTIONS[args.workload], "inputs": "seeded N(0,1) rounded "
                    "to bf16", "output": "e4m3fn codes + fp32 power-of-two scale per 1x128",
                    "parallelism": "single GPU", "rotation_copies": copies, "timing": args.timing}
                   if args.workload == "quant" else
                   {"workload": DESCRIPTIONS[args.workload].replace(" NT ", f" {args.layout.upper()} "),
                    "inputs": "seeded N(0,1) quantized to "
                    "e4m3fn, A per 1x128, B per 128x128, power-of-two scales",
                    "sfa_layout": "packed UE8M0" if args.sfa == "ue8m0" else "fp32",
                    "operand_layout": args.layout.upper(),
                    "accumulate": "fp32",
                    "output": ("e4m3fn codes + fp32 scale per 1x128 of silu(gate) * up"
                               if args.workload == "moe_swiglu" else "bf16"),
                    "parallelism": "single GPU",
                    "rotation_copies": copies,
                    "timing": args.timing}),
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kern,
        **line_extra,
        "wall_s": wall,
        "build_id": dg.BUILD_ID,
    }
    print(json.dumps(line), flush=True)


def mfma_ceiling(iters: int = 2000, reps: int = 10):
    """The matrix-instruction rate probe (libdg_probe.so): one workgroup of 8 waves per
    CU, each wave 4 * iters FP8 32x32x64 MFMAs on random e4m3fn register operands,
    graph-timed, with the gfx clock sampled meanwhile: (TFLOP/s, GHz or None)."""
    import ctypes
    import torch
    from fp8_block_scaled_dg_amd import build as dgb
    lib = ctypes.CDLL(dgb.PROBE_LIB_PATH)
    lib.dg_probe_mfma_rate.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                       ctypes.c_void_p, ctypes.c_void_p]
    blocks = 256
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda:0")

    def launch(i):
        rc = lib.dg_probe_mfma_rate(iters, blocks, 12345 + i, sink.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
        assert rc == 0, rc
    for i in range(3):
        launch(i)
    torch.cuda.synchronize()
    sampler = ClockSampler()
    ms = timed_launches(launch, reps, 0, True, sampler)
    flops = blocks * 8 * 4 * iters * 2.0 * 32 * 32 * 64
    mhz = sampler.mean()
    return flops / (ms * 1e-3) / 1e12, (mhz / 1e3 if mhz else None)


def overlap_probe(iters: int = 400, rounds: int = 5) -> dict:
    """The overlap probe (libdg_probe.so): per iteration each of 8 waves per CU issues
    six 1 KB global->LDS DMAs and eight FP8 32x32x64 MFMAs, as the compute-bound kernel
    does per K-block; modes: MFMA alone, DMA alone, both independent, MFMAs fed from the
    DMA'd LDS stages (fragments read an iteration ahead), and that plus a wait, a barrier
    and the promotion FMAs per iteration. Operand regions of 4 MB (L2-resident) and
    64 MB (streamed from MALL); modes interleaved over `rounds`, median ns per iteration."""
    import ctypes
    import torch
    from fp8_block_scaled_dg_amd import build as dgb
    lib = ctypes.CDLL(dgb.PROBE_LIB_PATH)
    lib.dg_probe_overlap.argtypes = [ctypes.c_int32, ctypes.c_void_p, ctypes.c_int64,
                                     ctypes.c_int32, ctypes.c_int32, ctypes.c_uint32,
                                     ctypes.c_void_p, ctypes.c_void_p]
    blocks = 256
    sink = torch.empty(blocks * 512, dtype=torch.float32, device="cuda:0")
    modes = {0: "mfma", 1: "dma", 2: "mfma+dma", 3: "mfma on lds fragments (read ahead)",
             4: "+ wait, barrier, promotion"}
    regions = {mb: torch.randint(0, 256, (mb << 20,), dtype=torch.uint8, device="cuda:0")
               for mb in (4, 64)}
    res = {}
    for r in range(rounds):
        for mb, buf in regions.items():
            for m in modes:
                def launch(i, m=m, buf=buf, mb=mb):
                    rc = lib.dg_probe_overlap(m, buf.data_ptr(), mb << 20, iters, blocks,
                                              777 + i, sink.data_ptr(),
                                              torch.cuda.current_stream().cuda_stream)
                    assert rc == 0, rc
                if r == 0:
                    launch(0)
                    torch.cuda.synchronize()
                ms = timed_launches(launch, 5, 0, graph=True)
                res.setdefault((mb, m), []).append(ms * 1e6 / iters)
    out = {}
    for (mb, m), v in sorted(res.items()):
        v = sorted(v)
        out.setdefault(f"{mb}MB", {})[modes[m]] = v[len(v) // 2]
    return out


def vendor_gemm(names, K: int, rotate: int, graph: bool) -> dict:
    """A reference point, not this library: the vendor FP8 GEMM (torch._scaled_mm, which
    calls hipBLASLt) on the named dense workloads with the same e4m3fn codes, with one
    scale per tensor and with one scale per row of A and per column of B. Neither form
    applies a scale per 128-wide K-block, so it computes a different product and its
    output is not checked; it shows what a tuned FP8 GEMM without per-block promotion
    reaches on this GPU. Inputs rotate like this library's legs; graph: the K launches
    are replayed from a HIP graph (the decode shapes, whose kernels are shorter than a
    host launch), else launched eagerly (prefill, where the launch gap is negligible)."""
    import torch
    import synth
    dev = "cuda:0"
    fp8 = torch.float8_e4m3fn
    out = {}
    for name in names:
        w = synth.workload(name)
        M, N, Kd = w.shape[:3]
        footprint = M * Kd + N * Kd + 2 * M * N
        copies = max(1, min(MAX_COPIES, -(-rotate // footprint)))
        A0 = torch.from_numpy(w.A).to(dev).view(fp8)
        B0 = torch.from_numpy(w.B).to(dev).view(fp8)
        sets = [dict(A=A0.clone(), B=B0.clone(),
                     C=torch.empty(M, N, dtype=torch.bfloat16, device=dev))
                for _ in range(copies)]
        del A0, B0
        forms = {"per_tensor": (torch.ones((), device=dev), torch.ones((), device=dev)),
                 "rowwise": (torch.ones(M, 1, device=dev), torch.ones(1, N, device=dev))}
        res = {}
        for form, (sa, sb) in forms.items():
            def launch(i, sa=sa, sb=sb):
                st = sets[i % copies]
                torch._scaled_mm(st["A"], st["B"].t(), sa, sb, out_dtype=torch.bfloat16,
                                 out=st["C"])
            t0 = time.perf_counter()
            i = 0
            while time.perf_counter() - t0 < 0.5 or i < 20:
                launch(i)
                i += 1
                if i % 20 == 0:
                    torch.cuda.synchronize()
            torch.cuda.synchronize()
            ms = timed_launches(launch, K, i, graph)
            res[form] = dict(avg_us=ms * 1e3, tflops=2.0 * M * N * Kd / (ms * 1e-3) / 1e12,
                             gbs=(M * Kd + N * Kd + 2 * M * N) / (ms * 1e-3) / 1e9)
        out[name] = dict(shape=dict(M=M, N=N, K=Kd), rotation_copies=copies, forms=res)
    return out


def vendor_prefill(K: int, rotate: int) -> dict:
    """The vendor reference on the prefill shape 4096x7168x18432 (see vendor_gemm)."""
    r = vendor_gemm(["prefill"], K, rotate, False)["prefill"]
    best = max(r["forms"].values(), key=lambda d: d["tflops"])
    return {"metric": "vendor FP8 GEMM TFLOPS on 4096x7168x18432 (reference point)",
            "value": best["tflops"], "unit": "TFLOPS", "n_gpus": 1, "steps": K,
            "higher_is_better": True, "dtype": "fp8", "data": "synthetic",
            "config": {"workload": "torch._scaled_mm (hipBLASLt), e4m3fn operands, bf16 "
                       "output, no per-128-K scaling", "rotation_copies": r["rotation_copies"],
                       "timing": "eager"},
            "forms": r["forms"]}


def vendor_decode(K: int, rotate: int) -> dict:
    """The vendor reference on the decode shapes 64x2112x7168 and 64x32768x512 (see
    vendor_gemm), graph-replayed like this library's decode step; bytes are the operand
    and output bytes (no scales), GB/s against the same 8 TB/s."""
    r = vendor_gemm(["dec2112", "dec32768"], K, rotate, True)
    best = {n: min(v["forms"].values(), key=lambda d: d["avg_us"]) for n, v in r.items()}
    total_bytes = sum(DECODE_BYTES.values())
    step_us = sum(b["avg_us"] for b in best.values())
    return {"metric": "vendor FP8 GEMM GB/s on the decode pair (reference point)",
            "value": total_bytes / (step_us * 1e-6) / 1e9, "unit": "GB/s", "n_gpus": 1,
            "steps": K, "higher_is_better": True, "dtype": "fp8", "data": "synthetic",
            "config": {"workload": "torch._scaled_mm (hipBLASLt), e4m3fn operands, bf16 "
                       "output, no per-128-K scaling; 64x2112x7168 + 64x32768x512",
                       "timing": "graph"},
            "gemms": r}


def prefill_leg(K: int, rotate: int, graph: bool) -> dict:
    """The compute-bound half of the metric: the dense prefill GEMM 4096x7168x18432,
    K launches timed like the step's GEMMs, against the dense FP8 MFMA peak; the shader
    clock sampled during the timed launches gives the peak at the clock the chip ran.
    The last launch's output is checked against the oracle on seeded whole rows."""
    import numpy as np
    import torch
    import synth
    g = Gemm("prefill", synth.workload("prefill"))
    copies = max(1, min(MAX_COPIES, -(-rotate // g.footprint)))
    g.upload(copies)
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < 0.5 or i < 20:
        g.launch(i)
        i += 1
        if i % 20 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    sampler = ClockSampler()
    ms = timed_launches(g.launch, K, i, graph, sampler)
    tflops = g.flops / (ms * 1e-3) / 1e12
    mhz = sampler.mean()
    roof = dict(bound="mfma", achieved=tflops, peak=FP8_PEAK_TFLOPS, unit="TFLOP/s",
                frac=tflops / FP8_PEAK_TFLOPS, kernel="prefill",
                clock_ghz=(mhz / 1e3) if mhz else None,
                peak_at_clock=(FP8_PEAK_TFLOPS * mhz / 1e3 / PEAK_CLOCK_GHZ) if mhz else None,
                frac_at_clock=(tflops / (FP8_PEAK_TFLOPS * mhz / 1e3 / PEAK_CLOCK_GHZ))
                if mhz else None,
                clock_samples=len(sampler.samples))
    ceil_tf, ceil_ghz = mfma_ceiling()
    roof.update(ceiling_tflops=ceil_tf, ceiling_clock_ghz=ceil_ghz,
                frac_of_ceiling=tflops / ceil_tf)
    # parity of the last timed launch on seeded whole rows
    import oracle
    from tests.parity import report
    w = g.w
    rows = np.sort(np.random.default_rng(4321).choice(w.shape[0], 32, replace=False))
    N = w.shape[1]
    ri = np.repeat(rows, N).astype(np.int64)
    ni = np.tile(np.arange(N, dtype=np.int64), rows.size)
    r = oracle.gemm_nt_at(w.A, w.B, w.sfA, w.sfB, ri, ni)
    C = g.sets[(i + K - 1) % len(g.sets)]["C"].view(torch.int16).cpu().numpy().view(np.uint16)
    rep = report(C[ri, ni], r)
    out = dict(shape=g.shape, launches=K, avg_us=ms * 1e3, tflops=tflops, alg_flops=g.flops,
               alg_bytes=g.bytes, rotation_copies=copies,
               parity={k: rep[k] for k in ("n", "max_excess_rel", "bitwise_match", "n_fail", "nan")},
               roofline=roof)
    del g
    torch.cuda.empty_cache()
    return {"prefill": out}


def copy_calibration(nbytes: int = 256 * 1024 * 1024, reps: int = 5):
    """A plain device-to-device copy of known size: under rocprofv3 --pmc its
    FETCH_SIZE / WRITE_SIZE per dispatch calibrate the HBM-traffic counters."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": nbytes, "reps": reps}), flush=True)


def measured_traffic(kernel_name: str, build_id: str):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary, if it was taken on the library build now loaded; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("build_id") != build_id:
        return None
    return rec.get("bytes_per_launch", {}).get(kernel_name)


# ---------------------------------------------------------------- profile summaries
#
# A manifest (JSON) lists rocprofv3 output folders and the exact commands that made
# them:
#   {"trace": [{"label": "decode", "dir": ..., "bench_json": ..., "command": ...}],
#    "traffic": {"calibration": {"fetch": DIR, "write": DIR, "command_fetch": ...,
#                                "command_write": ...},
#                "gemms": [{"gemm": "dec2112", "workload": "decode", "fetch": DIR,
#                           "write": DIR, "command_fetch": ..., "command_write": ...,
#                           "bench_fetch": OUT, "bench_write": OUT}]}}
# (bench_fetch / bench_write: the counter runs' stdout, whose bench line names the
# library build the counters were taken on)
# and --summarize turns them into short text summaries under profiles/.

def _csv_rows(folder: str, suffix: str):
    import csv
    import glob
    if not os.path.isabs(folder):
        folder = os.path.join(ROOT, folder)
    paths = sorted(glob.glob(os.path.join(folder, "**", "*" + suffix), recursive=True))
    if not paths:
        raise FileNotFoundError(f"no *{suffix} under {folder}")
    with open(paths[0]) as f:
        return list(csv.DictReader(f))


PROBE_KERNELS = ("stream_read_kernel", "mfma_rate_kernel", "empty_kernel")


def _ours(name: str) -> bool:
    return "dg::" in name


def _short(name: str) -> str:
    return name.replace("void ", "").split("(")[0]


def _per_dispatch(folder: str, counter: str):
    """counter value per dispatch of each of our kernels, averaged over dispatches."""
    acc, disp = {}, {}
    for r in _csv_rows(folder, "counter_collection.csv"):
        if r["Counter_Name"] != counter:
            continue
        k = r["Kernel_Name"]
        acc[k] = acc.get(k, 0.0) + float(r["Counter_Value"])
        disp.setdefault(k, set()).add(r["Dispatch_Id"])
    return {k: acc[k] / len(disp[k]) for k in acc}, {k: len(v) for k, v in disp.items()}


def _summarize_counters(entries, out_dir: str) -> None:
    """MFMA busy fraction per compute-bound workload from SQ_VALU_MFMA_BUSY_CYCLES
    (summed over every SIMD; 64 per 32x32x64 FP8 MFMA) and GRBM_GUI_ACTIVE (summed
    over the XCCs), averaged over our kernel's dispatches."""
    agent = [r for r in _csv_rows(entries[0]["dir"], "agent_info.csv") if r["Agent_Type"] == "GPU"][0]
    simds, xcc = int(agent["Simd_Count"]), int(agent["Num_Xcc"])
    clk = float(agent["Max_Engine_Clk_Fcompute"]) / 1e3
    md = ["# MFMA utilisation (rocprofv3 SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE)", "",
          f"GPU: {agent['Name']}, {simds} SIMDs, {xcc} XCCs, {clk:.1f} GHz peak engine clock. "
          "busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE per XCC x SIMDs), the rocprofv3 "
          "MfmaUtil expression; MFMAs = busy cycles / 64 (one 32x32x64 FP8 MFMA keeps a SIMD's "
          "matrix unit busy 64 cycles); clock = GRBM_GUI_ACTIVE per XCC / dispatch duration; "
          "busy x clock / peak clock is the fraction of the FP8 peak the MFMA work reaches. "
          "GRBM_GUI_ACTIVE spans slightly more than the kernel (launch and drain), so the clock "
          "reads a little high on the shorter kernels.", "",
          "| workload | dispatches | MFMAs issued | algorithmic MFMAs | busy | clock GHz | busy x clock/peak |",
          "|---|---|---|---|---|---|---|"]
    for e in entries:
        rows = [r for r in _csv_rows(e["dir"], "counter_collection.csv") if _ours(r["Kernel_Name"])]
        val, disp, dur = {}, set(), {}
        for r in rows:
            val.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            disp.add(r["Dispatch_Id"])
            dur[r["Dispatch_Id"]] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e9
        busy = sum(val["SQ_VALU_MFMA_BUSY_CYCLES"]) / len(val["SQ_VALU_MFMA_BUSY_CYCLES"])
        gui = sum(val["GRBM_GUI_ACTIVE"]) / len(val["GRBM_GUI_ACTIVE"]) / xcc
        t = sum(dur.values()) / len(dur)
        util = busy / (gui * simds)
        ghz = gui / t / 1e9
        bj = e["dir"] + ".json"
        bj = bj if os.path.isabs(bj) else os.path.join(ROOT, bj)
        with open(bj) as f:
            line = json.loads([x for x in f.read().splitlines() if x.startswith("{")][-1])
        alg = sum(k["alg_flops"] for k in line["kernels"]) / (2 * 32 * 32 * 64)
        md.append(f"| {e['label']} | {len(disp)} | {busy / 64:.4g} | {alg:.4g} | {util:.3f} | "
                  f"{ghz:.2f} | {util * ghz / clk:.3f} |")
    md += ["", "Commands (repository root on the GPU host):", ""]
    md += ["    " + e["command"] for e in entries]
    with open(os.path.join(out_dir, "counters_mfma.md"), "w") as f:
        f.write("\n".join(md) + "\n")


def _summarize_operand_path(passes, out_dir: str) -> None:
    """Where the compute-bound kernel's cycles go on the operand path: TA (address) and
    TD (data return) busy per CU, TD stalled on the texture cache, wave-cycles spent in
    s_waitcnt, LDS bank conflicts; counters averaged over our kernel's dispatches and
    normalised by GRBM_GUI_ACTIVE per XCC."""
    agent = [r for r in _csv_rows(passes[0]["dir"], "agent_info.csv") if r["Agent_Type"] == "GPU"][0]
    cus, xcc, ses = int(agent["Cu_Count"]), int(agent["Num_Xcc"]), int(agent["Num_Shader_Banks"])
    vals = {}
    for e in passes:
        d = {}
        for r in _csv_rows(e["dir"], "counter_collection.csv"):
            if _ours(r["Kernel_Name"]):
                d.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for k, v in d.items():
            vals.setdefault(e["label"], {})[(e["pass"], k)] = sum(v) / len(v)
    md = ["# Operand path of the compute-bound kernel (rocprofv3 TA / TD / SQ counters)", "",
          f"Per-CU blocks are normalised by GRBM_GUI_ACTIVE per XCC x {cus} CUs, the LDS command "
          f"FIFO by GRBM_GUI_ACTIVE per XCC x {ses} shader engines; wave figures are fractions of "
          "SQ_WAVE_CYCLES (both in quad-cycles), bank conflicts a fraction of SQ_LDS_IDX_ACTIVE.", "",
          "| workload | TA busy | TD busy | TD stalled on TC | waves in s_waitcnt | waves waiting on LDS | "
          "LDS cmd FIFO full | LDS bank conflicts |", "|---|---|---|---|---|---|---|---|"]
    for wl, v in vals.items():
        gui = v[("B", "GRBM_GUI_ACTIVE")] / xcc
        per_cu = lambda k: v[("B", k)] / (gui * cus)
        wave = v[("A", "SQ_WAVE_CYCLES")]
        md.append(f"| {wl} | {per_cu('TA_TA_BUSY_sum'):.2f} | {per_cu('TD_TD_BUSY_sum'):.2f} | "
                  f"{per_cu('TD_TC_STALL_sum'):.2f} | {v[('A', 'SQ_WAIT_INST_ANY')] / wave:.2f} | "
                  f"{v[('A', 'SQ_WAIT_INST_LDS')] / wave:.2f} | "
                  f"{v[('B', 'SQ_LDS_CMD_FIFO_FULL')] / (gui * ses):.2f} | "
                  f"{v[('A', 'SQ_LDS_BANK_CONFLICT')] / v[('A', 'SQ_LDS_IDX_ACTIVE')]:.3f} |")
    md += ["", "Commands (repository root on the GPU host):", ""]
    md += ["    " + e["command"] for e in passes]
    with open(os.path.join(out_dir, "counters_operand_path.md"), "w") as f:
        f.write("\n".join(md) + "\n")


INSTMIX = ("SQ_INSTS_VALU", "SQ_INSTS_MFMA", "SQ_INSTS_VALU_FMA_F32", "SQ_INSTS_LDS",
           "SQ_INSTS_VMEM", "SQ_INSTS_SALU", "SQ_INSTS_VALU_MFMA_F8", "SQ_INSTS_VALU_MFMA_F6F4")


def _summarize_instmix(entries, out_dir: str) -> None:
    """Wave-instruction mix of our kernel per workload (SQ_INSTS_*: each wave
    instruction counted once, summed over the GPU), averaged over its dispatches. The
    promotion is one fp32 FMA per accumulator element and K-block, i.e. M_v * N * KB / 64
    wave instructions; the table sets the FMAs counted against that and against the
    MFMAs (MFMA counts VALU-class instructions too: the other VALU is VALU - MFMA - FMA)."""
    md = ["# Instruction mix (rocprofv3 SQ_INSTS_*)", "",
          "Wave instructions per launch of our kernel (one count per wave instruction, summed "
          "over every wave), averaged over its dispatches. Promotion FMAs: the algorithmic count "
          "is one fp32 FMA per output element and K-block, M_v x N x K/128 / 64 wave "
          "instructions.", "",
          "| workload | MFMA | fp32 FMA | promotion FMAs (algorithmic) | FMA per MFMA | other VALU | "
          "LDS | VMEM | SALU |", "|---|---|---|---|---|---|---|---|---|"]
    for e in entries:
        v = {c: _per_dispatch(e["dir"], c)[0] for c in INSTMIX}
        ks = [k for k in v["SQ_INSTS_MFMA"] if _ours(k)]
        if len(ks) != 1:
            raise RuntimeError(f"{e['label']}: expected one of our kernels, got {ks}")
        k = ks[0]
        g = {c: v[c].get(k, 0.0) for c in INSTMIX}
        bj = e["dir"] + ".json"
        bj = bj if os.path.isabs(bj) else os.path.join(ROOT, bj)
        with open(bj) as f:
            line = json.loads([x for x in f.read().splitlines() if x.startswith("{")][-1])
        alg = sum(kk["alg_flops"] / 2 / 128 / 64 for kk in line["kernels"])
        mfma = g["SQ_INSTS_MFMA"]
        other = g["SQ_INSTS_VALU"] - mfma - g["SQ_INSTS_VALU_FMA_F32"]
        md.append(f"| {e['label']} | {mfma:.4g} | {g['SQ_INSTS_VALU_FMA_F32']:.4g} | {alg:.4g} | "
                  f"{g['SQ_INSTS_VALU_FMA_F32'] / max(mfma, 1):.2f} | {other:.4g} | "
                  f"{g['SQ_INSTS_LDS']:.4g} | {g['SQ_INSTS_VMEM']:.4g} | {g['SQ_INSTS_SALU']:.4g} |")
    md += ["", "Commands (repository root on the GPU host):", ""]
    md += ["    " + e["command"] for e in entries]
    with open(os.path.join(out_dir, "counters_instmix.md"), "w") as f:
        f.write("\n".join(md) + "\n")


def summarize(manifest_path: str) -> None:
    with open(manifest_path) as f:
        man = json.load(f)
    out_dir = os.path.join(ROOT, "profiles")
    os.makedirs(out_dir, exist_ok=True)
    timed = {}  # workload -> kernel -> timed-region average us
    for t in man.get("trace", []):
        stats = [r for r in _csv_rows(t["dir"], "kernel_stats.csv") if _ours(r["Name"])]
        bj = t["bench_json"] if os.path.isabs(t["bench_json"]) else os.path.join(ROOT, t["bench_json"])
        with open(bj) as f:
            line = json.loads([x for x in f.read().splitlines() if x.startswith("{")][-1])
        lines = [f"# Kernel trace: {line['config']['workload']}", "",
                 "Command (repository root on the GPU host):", "",
                 "    " + t["command"], "",
                 "rocprofv3 --stats, our kernels (all dispatches, warm-up included):", "",
                 "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
        for r in stats:
            lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | "
                         f"{float(r['AverageNs']) / 1e3:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                         f"{float(r['MaxNs']) / 1e3:.2f} |")
        # the timed region is each GEMM's last `steps` dispatches, launched back to back
        trace = [r for r in _csv_rows(t["dir"], "kernel_trace.csv") if _ours(r["Kernel_Name"])]
        per = {}
        for r in trace:
            per.setdefault(_short(r["Kernel_Name"]), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        K = line["steps"]
        lines += ["", f"Kernel trace of the timed region only (each kernel's last {K} "
                      "dispatches); `span` is first start to last end over the dispatches, "
                      "the launch-to-launch time:", "",
                  "| kernel | dispatches | avg us | median us | span us per dispatch |",
                  "|---|---|---|---|---|"]
        for k, ts in per.items():
            ts.sort()
            last = ts[-K:]
            avg = sum(e - s for s, e in last) / len(last) / 1e3
            med = sorted(e - s for s, e in last)[len(last) // 2] / 1e3
            span = (last[-1][1] - last[0][0]) / len(last) / 1e3
            lines.append(f"| `{k}` | {len(last)} | {avg:.2f} | {med:.2f} | {span:.2f} |")
            timed.setdefault(t["label"], {})[k] = avg
        probes = {}
        for r in _csv_rows(t["dir"], "kernel_trace.csv"):
            name = r["Kernel_Name"]
            tag = next((p for p in PROBE_KERNELS if p in name), None)
            if tag is None:
                continue
            if "<true>" in name:
                tag += " (non-temporal)"
            wgs = int(r["Grid_Size_X"]) // max(1, int(r["Workgroup_Size_X"]))
            probes.setdefault((tag, wgs), []).append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"])))
        if probes:
            # the streaming reads run byte count by byte count (outer loop), in the order
            # of the line's hbm_ceiling entries
            sizes = [int(k) for k in (line.get("hbm_ceiling") or {}) if k.isdigit()]
            lines += ["", "Calibration probes of the same run (libdg_probe.so), kernel time; "
                          "bench.py graph-times them itself and reports the best streaming-read "
                          "configuration per byte count:", "",
                      "| probe | bytes | workgroups | dispatches | min us | median us |",
                      "|---|---|---|---|---|---|"]
            for (tag, wgs), d in sorted(probes.items()):
                d.sort()
                parts = [(None, d)]
                if tag.startswith("stream_read") and sizes and len(d) % len(sizes) == 0:
                    n = len(d) // len(sizes)
                    parts = [(sizes[i], d[i * n:(i + 1) * n]) for i in range(len(sizes))]
                for nbytes, seg in parts:
                    us = sorted((e - s0) / 1e3 for s0, e in seg)
                    lines.append(f"| `{tag}` | {nbytes or ''} | {wgs} | {len(us)} | "
                                 f"{us[0]:.2f} | {us[len(us) // 2]:.2f} |")
        lines += ["", "bench.py line of the same run (HIP events around each GEMM's "
                      "back-to-back launches):", ""]
        for k in line["kernels"]:
            lines.append(f"- {k['name']} {k['shape']}: {k['avg_us']:.2f} us per launch")
        lines += [f"- value: {line['value']:.1f} {line['unit']}, "
                  f"roofline frac {line['roofline']['frac']:.3f}", ""]
        with open(os.path.join(out_dir, f"trace_{t['label']}.md"), "w") as f:
            f.write("\n".join(lines))
    cn = man.get("counters")
    if cn:
        _summarize_counters(cn, out_dir)
    ps = man.get("passes")
    if ps:
        _summarize_operand_path(ps, out_dir)
    im = man.get("instmix")
    if im:
        _summarize_instmix(im, out_dir)
    tr = man.get("traffic")
    if tr:
        cal = tr["calibration"]
        cf, _ = _per_dispatch(cal["fetch"], "FETCH_SIZE")
        cw, _ = _per_dispatch(cal["write"], "WRITE_SIZE")
        # the largest copy kernel in the calibration run is the 256 MiB copy
        copy_kib = 256 * 1024
        k_f = max(((v, k) for k, v in cf.items() if "copy" in k.lower() or "elementwise" in k),
                  default=None)
        if k_f is None:
            k_f = max((v, k) for k, v in cf.items())
        kern = k_f[1]
        f_scale = copy_kib / cf[kern]
        w_scale = copy_kib / cw[kern]
        # the library build the counters were taken on: the build id on the bench lines of
        # the counter runs themselves (every run must agree)
        ids = set()
        for g in tr["gemms"]:
            for key in ("bench_fetch", "bench_write"):
                bj = g[key] if os.path.isabs(g[key]) else os.path.join(ROOT, g[key])
                with open(bj) as f:
                    ids.add(json.loads([x for x in f.read().splitlines()
                                        if x.startswith("{")][-1])["build_id"])
        if len(ids) != 1:
            raise RuntimeError(f"counter runs on different library builds: {sorted(ids)}")
        rec = {"build_id": ids.pop(),
               "calibration": {"kernel": _short(kern), "copy_bytes": copy_kib * 1024,
                               "fetch_kib": cf[kern], "write_kib": cw[kern],
                               "fetch_scale": f_scale, "write_scale": w_scale,
                               "command_fetch": cal["command_fetch"],
                               "command_write": cal["command_write"]},
               "bytes_per_launch": {}, "detail": {}}
        md = ["# HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)", "",
              "Calibration: a plain 256 MiB device copy reads "
              f"{cf[kern]:.0f} KiB and writes {cw[kern]:.0f} KiB per dispatch "
              f"(kernel `{_short(kern)}`); scale factors fetch {f_scale:.4f}, "
              f"write {w_scale:.4f}.", "",
              "    " + cal["command_fetch"], "    " + cal["command_write"], "",
              "| GEMM | kernel | dispatches | fetch KiB | write KiB | scaled bytes | kernel us | HBM GB/s |",
              "|---|---|---|---|---|---|---|---|"]
        for g in tr["gemms"]:
            fv, fn = _per_dispatch(g["fetch"], "FETCH_SIZE")
            wv, _ = _per_dispatch(g["write"], "WRITE_SIZE")
            ours = [k for k in fv if _ours(k)]
            if len(ours) != 1:
                raise RuntimeError(f"{g['gemm']}: expected one of our kernels, got {ours}")
            k = ours[0]
            b = fv[k] * f_scale * 1024 + wv.get(k, 0.0) * w_scale * 1024
            rec["bytes_per_launch"][g["gemm"]] = b
            rec["detail"][g["gemm"]] = {"kernel": _short(k), "fetch_kib": fv[k],
                                        "write_kib": wv.get(k, 0.0), "dispatches": fn[k],
                                        "command_fetch": g["command_fetch"],
                                        "command_write": g["command_write"]}
            us = timed.get(g["workload"], {}).get(_short(k))
            rate = f"{us:.1f} | {b / (us * 1e-6) / 1e9:.0f}" if us else "- | -"
            md.append(f"| {g['gemm']} | `{_short(k)}` | {fn[k]} | {fv[k]:.0f} | "
                      f"{wv.get(k, 0.0):.0f} | {b:.4g} | {rate} |")
            md += ["", "    " + g["command_fetch"], "    " + g["command_write"], ""]
        md.append("kernel us: the kernel trace's timed-region average of the same workload "
                  "(trace_*.md); HBM GB/s: scaled bytes / kernel us, the rate the L2 misses and "
                  "write-backs reach (partials of split-K included), against 8 TB/s.")
        md.append("")
        md.append(f"library build id: {rec['build_id']}")
        with open(os.path.join(out_dir, "traffic.json"), "w") as f:
            json.dump(rec, f, indent=1)
        with open(os.path.join(out_dir, "traffic.md"), "w") as f:
            f.write("\n".join(md) + "\n")


if __name__ == "__main__":
    main()
