#!/usr/bin/env python3
"""HGRNBit layer throughput on one MI355X: prefill + decode at the 1.3B shape.

One step is one serving pass over one batch of seeded synthetic input through
a 24-layer HGRNBit stack (d=2048, MLP inner 5632, random ternarised weights):
  1. prefill: B sequences of T prompt tokens through every layer (chunked scan);
  2. decode: D tokens per sequence, one layer step at a time, each continuing
     from the state the prefill left in that layer (a HIP graph per token step).
value = layer-tokens/s = B*(T+D)*L / step time (metric "HGRNBit layer tokens/s").

Also printed in the same JSON line:
  roofline     -- the dominant kernel at its shape (largest share of the step
                  time) against its roof: int8 MFMA peak for a prefill
                  contraction, HBM for everything else. Kernels are timed by
                  HIP events recorded around each launch on its stream:
                  prefill kernels inside the timed steps; decode kernels, which
                  run inside a HIP graph there, on an eager copy of the decode
                  steps queued behind a prefill. Where profiles/ holds a
                  rocprofv3 kernel trace of the same sources, that kernel's
                  trace average is printed beside the event figure;
  cpu_baseline -- the CPU oracle on a bounded sample of the same workload;
  configs      -- with --extras (default): every other config of the workload
                  (370M layer fp32; 370M and 2.7B stack prefills; the 1.3B
                  decode step at batch 1, 16, 64; the long-sequence scan; the
                  expanded-state recurrence, prefill and decode step; the
                  decode GEMV streaming 67 and 268 MB of weights), each
                  with its own roofline (the fp32 vector ALU for the
                  expanded-state prefill), next to a measured HBM ceiling.
--only LEG runs one config leg alone, for profiling it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
FP32_VECTOR_PEAK_TFLOPS = 157.3  # MI355X fp32 vector (packed, 256 CUs at 2.4 GHz)
FP32_MFMA_PEAK_TFLOPS = 157.3    # MI355X dense fp32 MFMA
INT8_MFMA_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--shape", default="1.3B", choices=["370M", "1.3B", "2.7B"])
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--prompt", type=int, default=2048)
    ap.add_argument("--decode", type=int, default=512)
    ap.add_argument("--cpu-baseline", type=int, default=1, help="0 skips the CPU oracle leg")
    ap.add_argument("--no-graph", action="store_true", help="launch decode steps eagerly instead of a HIP graph")
    ap.add_argument("--extras", type=int, default=1,
                    help="0 skips the figures measured outside the timed steps (the other configs, the "
                         "measured HBM ceiling, derivatives, generation)")
    ap.add_argument("--only", choices=["c1", "c2", "c3", "c4", "c5", "prefill_b8", "ceiling", "bwd", "hgrn2",
                                       "gemv"],
                    help="run one config leg alone and print its JSON (for profiling a config)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy three times (for scaling HBM counters)")
    ap.add_argument("--vendor-int8-gemm", action="store_true",
                    help="only time the vendor library's dense int8 GEMM (torch._int_mm) at the prefill "
                         "contraction shapes and its dense bf16 product at the decode shapes, as references")
    return ap.parse_args()


def calibrate_copy():
    """A plain copy of known size: what FETCH_SIZE / WRITE_SIZE read for it scales the counters
    of the library's kernels to bytes."""
    import torch
    n = 1 << 28
    a = torch.ones(n, device="cuda")
    b = torch.empty(n, device="cuda")
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    b.copy_(a)
    e0.record()
    for _ in range(2):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 2
    print(json.dumps({"copy_bytes_per_launch": 4 * n, "launches": 3, "us_per_launch": round(ms * 1000, 1),
                      "read_plus_write_GBps": round(8 * n / (ms / 1000) / 1e9, 1)}), flush=True)


def vendor_int8_gemm(shape: str, batch: int, prompt: int):
    """Dense int8 x int8 -> int32 products of the vendor library at the prefill shapes (weights as
    plain int8, no epilogue): what the same matrix cores reach without this library's kernels."""
    import torch
    from ternary_weight_matmul_amd import synth
    d, inner, _ = synth.SHAPES[shape]
    M = batch * prompt
    out = []
    for name, N, K in [("i/f/g", 3 * d, d), ("o_proj", d, d), ("gate_proj", 2 * inner, d), ("down_proj", d, inner)]:
        a = torch.randint(-127, 128, (M, K), dtype=torch.int8, device="cuda")
        b = torch.randint(-1, 2, (K, N), dtype=torch.int8, device="cuda")
        for _ in range(3):
            torch._int_mm(a, b)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch._int_mm(a, b)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 100.0
        tops = 2.0 * M * N * K / (us / 1e6) / 1e12
        out.append({"contraction": name, "m": M, "n": N, "k": K, "us": round(us, 1), "int8_tops": round(tops, 1),
                    "frac_mfma": round(tops / INT8_MFMA_PEAK_TOPS, 4)})
        del a, b
    # decode-shaped products (batch rows x dense bf16 weights): the same contractions as one
    # token step at this batch, with 16-bit instead of 2-bit weights
    dec = []
    for name, N, K in [("i/f/g", 3 * d, d), ("o_proj", d, d), ("gate_proj", 2 * inner, d), ("down_proj", d, inner)]:
        x = torch.randn(batch, K, device="cuda").to(torch.bfloat16)
        w = (torch.randn(N, K, device="cuda") * 0.02).to(torch.bfloat16)
        y = torch.nn.functional.linear(x, w)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()  # replayed, so that host launch cost does not count
        with torch.cuda.graph(g):
            for _ in range(20):
                y = torch.nn.functional.linear(x, w)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1000.0 / 100
        nbytes = 2.0 * (N * K + batch * K + batch * N)
        dec.append({"contraction": name, "m": batch, "n": N, "k": K, "us": round(us, 2),
                    "gbs": round(nbytes / (us / 1e6) / 1e9, 1), "frac_hbm": round(nbytes / (us / 1e6) / 1e9 / HBM_PEAK_GBS, 4)})
        del x, w, y, g
    print(json.dumps({"vendor_int8_gemm": out, "vendor_bf16_decode_linear": dec, "shape": shape}), flush=True)


ACT_BYTES = 2  # bf16 activations


def _kind(kernel: str):
    base, _, rest = kernel.partition("<")
    args = rest.rstrip(">").split(",") if rest else []
    return base, args


def algorithmic(kernel: str, m: int, n: int, k: int):
    """(ops, bytes) one launch must do at the least, from the kernel variant and its shape.

    contraction (m rows, n outputs over all groups, k): ops = 2 m n k; bytes = packed
      weights n k / 4 + int8 codes m k per activation tensor + scale and code sum 8 m per
      tensor + the epilogue's own traffic per output channel c of a group:
        gates: f, x~ and g written (fp32) = 12 B; gates_step: h read and written and g
        written (fp32) = 12 B; glu: z (fp32) = 4 B; resid: residual read and sum written, one
        fp32 and one bf16 = 6 B; linear: 4 B.
    tgemv_row<epi,T> (a contraction that quantises its own input rows): as a contraction, with
      the rows read once in type T (m k sizeof T) in place of the codes, scale and code sum;
      tgemv_row<resid,gnorm,T>: h (fp32) and g (T) per element and g_norm's gain (fp32) per k.
    norm_quant<T> (m rows of k): x read (sizeof T) + codes written (1 B) per element, 8 B per row.
    gnorm_quant<T>: h (fp32) and g (sizeof T) read + codes written per element, 8 B per row.
    scan (m = b t, k = d): f and x~ read, h written, 12 B per element.
    hgrn2_scan<e> / hgrn2_chunk<e> / hgrn2_step<e> (m = b t, n = d, k = e, the expanded-state
      recurrence, step-wise / chunked / one token): per token and head of e, 5 e^2 + e flops of
      the definition (the state's multiply, multiply-add and readout multiply-add, and 1 - f;
      the chunked form's own products are not counted); f, i, o read and y written, 16 B per
      (b, t, channel); a step (t = 1, m = b) also reads and writes the state, 8 e bytes per
      (b, channel).
    scan_bwd (m = b t, k = d): dh, f and h read, dx and df written, 20 B per element.
    """
    base, args = _kind(kernel)
    if base in ("hgrn2_scan", "hgrn2_step", "hgrn2_chunk"):
        e = int(args[0])
        nbytes = 16.0 * m * n + (8.0 * m * n * e if base == "hgrn2_step" else 0.0)
        return m * n * (5.0 * e + 1.0), nbytes
    if base in ("tgemm", "tgemm_dma", "tgemv", "tgemv_row"):
        epi = args[0]
        na = 3 if "split_a" in args else 1
        ng = {"gates": 3, "gates_step": 3, "glu": 2}.get(epi, 1)
        per_c = {"gates": 12, "gates_step": 12, "glu": 4, "resid": 4 + ACT_BYTES, "linear": 4}[epi]
        if base == "tgemv_row":
            tb = 4.0 if args[-1] == "f32" else ACT_BYTES
            # the gated g_norm reads h (fp32), g and g_norm's gain instead of x
            rows = m * k * (4.0 + tb) + 4.0 * k if "gnorm" in args else m * k * tb
        else:
            rows = na * (m * k + 8.0 * m)
        nbytes = n * k / 4.0 + rows + m * (n / ng) * per_c
        return 2.0 * m * n * k, nbytes
    tb = 4 if args[:1] == ["f32"] else ACT_BYTES
    if base == "norm_quant":
        return 0.0, m * k * (tb + 1.0) + 8.0 * m
    if base == "gnorm_quant":
        return 0.0, m * k * (4.0 + tb + 1.0) + 8.0 * m
    if base.startswith("scan_bwd"):
        return 0.0, 20.0 * m * k
    if base.startswith("scan"):
        return 0.0, 12.0 * m * k
    return 0.0, 0.0


# the source files each kernel family is built from
_COMMON = ["device_common.hpp", "launch.hpp"]
KERNEL_SOURCES = {
    "tgemv": ["k_contract.hip", "epilogue.hpp"] + _COMMON,
    "tgemv_row": ["k_contract.hip", "epilogue.hpp"] + _COMMON,
    "tgemm": ["k_contract.hip", "epilogue.hpp"] + _COMMON,
    "tgemm_dma": ["k_contract.hip", "epilogue.hpp"] + _COMMON,
    "norm_quant": ["k_quant.hip", "row_quant.hpp"] + _COMMON,
    "gnorm_quant": ["k_quant.hip", "row_quant.hpp"] + _COMMON,
    "scan": ["k_scan.hip"] + _COMMON,
    "hgrn2_scan": ["k_hgrn2.hip"] + _COMMON,
    "hgrn2_chunk": ["k_hgrn2.hip"] + _COMMON,
    "hgrn2_step": ["k_hgrn2.hip"] + _COMMON,
}


def kernel_files(kernel: str):
    base = _kind(kernel.split(" ")[0])[0]
    return KERNEL_SOURCES.get("scan" if base.startswith("scan") else base)


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed (what the compiler sees)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(files=None) -> str:
    """sha256 of kernel sources (the given files of csrc/, else all of them), comments and
    layout left out, to tell whether stored counter figures still apply to the code that runs."""
    import hashlib
    hsh = hashlib.sha256()
    csrc = os.path.join(ROOT, "ternary_weight_matmul_amd", "csrc")
    names = sorted(files) if files else sorted(n for n in os.listdir(csrc) if n.endswith((".hip", ".hpp")))
    for name in names:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            hsh.update(name.encode() + b"\0" + _code_only(f.read()).encode())
    return hsh.hexdigest()[:16]


def stored_traffic(key: str):
    """HBM bytes per launch of kernel `key` from a counter summary under profiles/ (FETCH_SIZE +
    WRITE_SIZE, scaled by the copy-kernel calibration), if one exists for the current sources of
    that kernel (the digest of the files it is built from)."""
    pdir = os.path.join(ROOT, "profiles")
    files = kernel_files(key)
    if not os.path.isdir(pdir) or not files:
        return None
    digest = source_digest(files)
    for name in sorted(os.listdir(pdir)):
        if not (name.startswith("traffic_") and name.endswith(".txt")):
            continue
        fields = {}
        with open(os.path.join(pdir, name)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    kk, _, vv = line.partition(":")
                    fields[kk.strip()] = vv.strip()
        if fields.get("kernel") == key and fields.get("sources") == digest:
            try:
                return float(fields["hbm_bytes_per_launch"])
            except (KeyError, ValueError):
                return None
    return None


class KernelTable:
    """Per-kernel totals from the library's timing records (events bound to each dispatch),
    keyed by variant and shape, with each launch's algorithmic ops and bytes."""

    def __init__(self):
        self.k = {}

    def add(self, recs, phase: str, scale: float):
        for name, m, n, k, ms in recs:
            key = "%s m=%d n=%d k=%d" % (name, m, n, k)
            e = self.k.setdefault(key, dict(name=name, m=m, n=n, k=k, phase=phase, launches=0.0, ms=0.0))
            e["launches"] += scale
            e["ms"] += ms * scale
        for e in self.k.values():
            e["avg_ms"] = e["ms"] / e["launches"]
            e["ops"], e["bytes"] = algorithmic(e["name"], e["m"], e["n"], e["k"])
        return self

    def total_ms(self, phase=None):
        return sum(e["ms"] for e in self.k.values() if phase is None or e["phase"] == phase)

    def dominant(self):
        return max(self.k.items(), key=lambda kv: kv[1]["ms"])

    def roofline(self, step_ms: float, key=None) -> dict:
        """The dominant kernel (or `key`) against its roof: the int8 MFMA peak for a prefill-shaped
        contraction, HBM for everything else; achieved = algorithmic work per launch / average
        launch duration."""
        key, e = (key, self.k[key]) if key else self.dominant()
        avg_s = e["avg_ms"] / 1000.0
        if e["name"].startswith("tgemm"):
            roof = dict(bound="mfma", achieved=round(e["ops"] / avg_s / 1e12, 2), peak=INT8_MFMA_PEAK_TOPS,
                        unit="TFLOP/s")
        elif e["name"].startswith("hgrn2_scan"):
            roof = dict(bound="alu", achieved=round(e["ops"] / avg_s / 1e12, 2), peak=FP32_VECTOR_PEAK_TFLOPS,
                        unit="TFLOP/s")
        elif e["name"].startswith("hgrn2_chunk"):
            roof = dict(bound="mfma", achieved=round(e["ops"] / avg_s / 1e12, 2), peak=FP32_MFMA_PEAK_TFLOPS,
                        unit="TFLOP/s")
        else:
            roof = dict(bound="hbm", achieved=round(e["bytes"] / avg_s / 1e9, 1), peak=HBM_PEAK_GBS, unit="GB/s")
        roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
        roof["traffic"] = stored_traffic(key)
        roof["kernel"] = key
        roof["phase"] = e["phase"]
        roof["avg_launch_us"] = round(e["avg_ms"] * 1000.0, 2)
        roof["launches_per_step"] = round(e["launches"], 1)
        roof["algorithmic_per_launch"] = e["ops"] if roof["bound"] in ("mfma", "alu") else e["bytes"]
        roof["share_of_step"] = round(e["ms"] / step_ms, 3)
        tr = stored_trace_us(key)
        if tr:  # the same kernel's average in a committed rocprofv3 trace of these sources
            us, fname = tr
            work = roof["algorithmic_per_launch"]
            roof["trace_avg_launch_us"] = us
            scale = 1e9 if roof["bound"] == "hbm" else 1e12
            roof["trace_frac"] = round(work / (us / 1e6) / scale / roof["peak"], 4)
            roof["trace_file"] = "profiles/" + fname
        return roof

    def contractions(self, phase: str = "prefill"):
        """All prefill-shaped contractions together against the int8 MFMA peak."""
        pre = [e for e in self.k.values() if e["phase"] == phase and e["name"].startswith("tgemm")]
        if not pre:
            return None
        ops = sum(e["ops"] * e["launches"] for e in pre)
        ms = sum(e["ms"] for e in pre)
        tops = ops / (ms / 1000) / 1e12
        return dict(achieved=round(tops, 1), peak=INT8_MFMA_PEAK_TOPS, unit="TFLOP/s",
                    frac=round(tops / INT8_MFMA_PEAK_TOPS, 4),
                    per_kernel={e["name"]: round(e["ops"] / (e["avg_ms"] / 1000) / 1e12 / INT8_MFMA_PEAK_TOPS, 4)
                                for e in pre})

    def breakdown(self, top: int = 0) -> dict:
        out = {}
        rows = sorted(self.k.items(), key=lambda kv: -kv[1]["ms"])
        for key, e in rows[:top] if top else rows:
            t = e["avg_ms"] / 1000.0
            row = dict(phase=e["phase"], launches_per_step=round(e["launches"], 1), avg_us=round(e["avg_ms"] * 1000, 2),
                       ms_per_step=round(e["ms"], 3))
            if e["ops"] and e["name"].startswith("hgrn2"):
                row["fp32_tflops"] = round(e["ops"] / t / 1e12, 2)
                if e["name"].startswith("hgrn2_chunk"):  # the chunked form runs on fp32 MFMA
                    row["frac_fp32_mfma"] = round(e["ops"] / t / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4)
                else:
                    row["frac_fp32_vector"] = round(e["ops"] / t / 1e12 / FP32_VECTOR_PEAK_TFLOPS, 4)
            elif e["ops"]:
                row["int8_tops"] = round(e["ops"] / t / 1e12, 1)
                row["frac_mfma"] = round(e["ops"] / t / 1e12 / INT8_MFMA_PEAK_TOPS, 4)
            row["gbs"] = round(e["bytes"] / t / 1e9, 1)
            row["frac_hbm"] = round(e["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4)
            if e["ops"] and not e["name"].startswith("hgrn2"):
                # the kernel against its own roof: the longer of its ops at the int8 MFMA peak and
                # its bytes at the HBM peak
                t_mfma = e["ops"] / (INT8_MFMA_PEAK_TOPS * 1e12)
                t_hbm = e["bytes"] / (HBM_PEAK_GBS * 1e9)
                row["own_roof"] = "mfma" if t_mfma >= t_hbm else "hbm"
                row["own_roof_us"] = round(max(t_mfma, t_hbm) * 1e6, 2)
                row["frac_own_roof"] = round(max(t_mfma, t_hbm) / t, 4)
            out[key] = row
        return out


def timed_records(mmf, fn, reps: int = 1):
    """Runs fn() reps times with the library's per-launch timing on; returns the records."""
    import torch
    torch.cuda.synchronize()
    mmf.timing_enable(True)
    for _ in range(reps):
        fn()
    torch.cuda.synchronize()
    mmf.timing_enable(False)
    return mmf.timing_collect()


def device_layers(mmf, torch, d: int, inner: int, L: int, seed: int, dev):
    """L blocks of random ternarised weights: latent weights ~ N(0, 0.02) drawn on the device
    (torch's generator seeded per layer with c*1000 + l), packed by mmf_ternary_pack."""
    shapes = {"i": (d, d), "f": (d, d), "g": (d, d), "o": (d, d), "gate": (2 * inner, d), "down": (d, inner)}
    layers = []
    gen = torch.Generator(device=dev)
    for l in range(L):
        gen.manual_seed(seed * 1000 + l)
        lat = {k: torch.randn(s_, device=dev, generator=gen) * 0.02 for k, s_ in shapes.items()}
        layers.append(mmf.LayerParams.pack(lat))
        del lat
    torch.cuda.synchronize()
    return layers


def event_ms(torch, fn, reps: int, warmup: int = 1):
    """Mean milliseconds of fn() over reps runs (events on the current stream), after warmup runs."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def hbm_ceilings(mmf, torch, dev, nbytes: int = 1 << 30, reps: int = 5) -> dict:
    """Measured HBM roof: mmf_hbm_ceiling's streaming read, copy, and two-reads-one-write of
    nbytes per stream."""
    src = torch.ones(nbytes // 2, device=dev)  # 2 * nbytes: the two read streams of 2r1w
    dst = torch.empty(nbytes // 4, device=dev)
    sink = torch.empty(32768, dtype=torch.uint8, device=dev)
    one = src[: nbytes // 4]

    def run():
        mmf.hbm_ceiling(one, sink, "read")
        mmf.hbm_ceiling(one, dst, "copy")
        mmf.hbm_ceiling(src, dst, "2r1w")

    run()
    recs = timed_records(mmf, run, reps)
    ms = {k: sum(r[4] for r in recs if r[0] == k) / reps for k in ("stream_read", "stream_copy", "stream_2r1w")}
    del src, dst, sink
    rd = nbytes / ms["stream_read"] / 1e6
    cp = 2 * nbytes / ms["stream_copy"] / 1e6
    r2 = 3 * nbytes / ms["stream_2r1w"] / 1e6
    return dict(bytes_per_stream=nbytes, read_GBs=round(rd, 1), copy_GBs=round(cp, 1), two_read_one_write_GBs=round(r2, 1),
                read_frac=round(rd / HBM_PEAK_GBS, 4), copy_frac=round(cp / HBM_PEAK_GBS, 4),
                two_read_one_write_frac=round(r2 / HBM_PEAK_GBS, 4),
                note="hand-written streaming kernels (mmf_hbm_ceiling): 256-thread workgroups each streaming a "
                     "contiguous range, 8 16-byte loads in flight per lane (read: 8192 workgroups, cached loads; "
                     "copy and 2r1w: 16384, non-temporal)")


def mfma_ceiling(mmf, torch, dev, iters: int = 16384, reps: int = 3) -> dict:
    """Measured int8 MFMA roof: mmf_mfma_ceiling's MFMA-only loop (four 256-thread workgroups per
    CU, four independent 32x32x32 int8 MFMA chains per wave), timed with events."""
    sink = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
    ops = mmf.mfma_ceiling(iters, sink)
    ms = event_ms(torch, lambda: mmf.mfma_ceiling(iters, sink), reps)
    del sink
    tops = ops / (ms / 1000.0) / 1e12
    return dict(int8_TOPs=round(tops, 1), frac=round(tops / INT8_MFMA_PEAK_TOPS, 4), ms_per_launch=round(ms, 3),
                note="MFMA-only loop (mmf_mfma_ceiling): v_mfma_i32_32x32x32_i8 on register operands, four "
                     "independent chains per wave, four waves per SIMD; the rate includes the clock the chip "
                     "holds under that load")


def with_ceiling(roof: dict, ceil: dict) -> dict:
    """An HBM-bound roof also read against the measured streaming roofs: the read stream for a
    contraction or quantiser, two reads and one write for the scan; an int8 contraction against
    the measured MFMA-only rate."""
    if ceil and roof.get("bound") == "hbm":
        roof["frac_of_measured_read"] = round(roof["achieved"] / ceil["read_GBs"], 4)
        roof["frac_of_measured_2r1w"] = round(roof["achieved"] / ceil["two_read_one_write_GBs"], 4)
    if ceil and ceil.get("mfma") and roof.get("bound") == "mfma" and roof.get("kernel", "").startswith("tgemm"):
        roof["frac_of_measured_mfma"] = round(roof["achieved"] / ceil["mfma"]["int8_TOPs"], 4)
    return roof


def contractions_with_ceiling(cr, ceil):
    """All prefill contractions together, also against the measured MFMA-only rate."""
    if cr and ceil and ceil.get("mfma"):
        cr["frac_of_measured_mfma"] = round(cr["achieved"] / ceil["mfma"]["int8_TOPs"], 4)
        cr["per_kernel_of_measured_mfma"] = {k: round(v * INT8_MFMA_PEAK_TOPS / ceil["mfma"]["int8_TOPs"], 4)
                                             for k, v in cr["per_kernel"].items()}
    return cr


def leg_prefill(mmf, torch, dev, shape: str, b: int, t: int, seed: int, reps: int, ceil=None) -> dict:
    """A whole-stack prefill of one config: L layers of `shape`, b x t bf16 tokens (x ~ N(0, 1)
    drawn on the device), scan mode auto; value = layer-tokens/s."""
    from ternary_weight_matmul_amd import synth
    d, inner, L = synth.SHAPES[shape]
    layers = device_layers(mmf, torch, d, inner, L, seed, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 10 + 1)
    x = torch.randn((b, t, d), device=dev, generator=gen).to(torch.bfloat16)
    bufs = [torch.empty_like(x) for _ in range(2)]
    hs = torch.empty((L, b, d), dtype=torch.float32, device=dev)
    ws = torch.empty(mmf.layer_workspace_size(layers[0], b, t), dtype=torch.uint8, device=dev)

    def run():
        cur = x
        for l in range(L):
            mmf.layer_fwd(layers[l], cur, None, out=bufs[l % 2], h_last=hs[l], ws=ws)
            cur = bufs[l % 2]

    ms = event_ms(torch, run, reps)
    kt = KernelTable().add(timed_records(mmf, run), "prefill", 1.0)
    del x, bufs, hs, ws, layers
    return dict(workload="%s stack prefill: %d layers d=%d inner=%d, bf16, B=%d x T=%d" % (shape, L, d, inner, b, t),
                value=round(b * t * L / (ms / 1000), 1), unit="layer-tokens/s", ms=round(ms, 3),
                stack_tokens_per_s=round(b * t / (ms / 1000), 1),
                roofline=with_ceiling(kt.roofline(ms), ceil),
                contraction_roofline=contractions_with_ceiling(kt.contractions(), ceil),
                kernels=kt.breakdown(8))


def leg_c1(mmf, torch, dev, reps: int = 100, cpu: bool = True) -> dict:
    """One 370M-width layer, fp32, batch 1 x 128 tokens, recurrent scan (the small config the
    oracle finishes in seconds): median of `reps` event-timed calls; the oracle timed on the same
    seeded host input and weights."""
    import numpy as np
    from ternary_weight_matmul_amd import synth
    d, inner, _ = synth.SHAPES["370M"]
    lat = synth.latent_weights(d, inner, synth.layer_seed(1, 0))
    P = mmf.LayerParams.pack({k: torch.from_numpy(v).to(dev) for k, v in lat.items()})
    xs = synth.activations((1, 128, d), 1)
    x = torch.from_numpy(xs).to(dev)
    out = torch.empty_like(x)
    ws = torch.empty(mmf.layer_workspace_size(P, 1, 128), dtype=torch.uint8, device=dev)

    def run():
        mmf.layer_fwd(P, x, None, out=out, ws=ws, mode="recurrent")

    for _ in range(5):
        run()
    torch.cuda.synchronize()
    times = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run()
        e1.record()
        e1.synchronize()
        times.append(e0.elapsed_time(e1))
    ms = float(np.median(times))
    kt = KernelTable().add(timed_records(mmf, run, 20), "prefill", 1.0 / 20)
    res = dict(workload="370M layer, fp32, B=1 x T=128, recurrent scan", value=round(128 / (ms / 1000), 1),
               unit="layer-tokens/s", ms_median=round(ms, 4), roofline=kt.roofline(ms), kernels=kt.breakdown(6),
               note="latency-bound: the whole layer is a few microseconds per kernel")
    if cpu:
        import oracle
        Lo = oracle.make_layer(lat)
        t0 = time.perf_counter()
        oracle.layer_forward(Lo, xs)
        dt = time.perf_counter() - t0
        res["cpu_oracle"] = dict(value=round(128 / dt, 2), unit="layer-tokens/s", cores=oracle.num_threads(),
                                 cpu=cpu_model(), sample="the whole config: 1 layer, 128 tokens (%.2f s)" % dt)
    return res


def leg_decode(mmf, torch, dev, batches=(1, 16, 64), steps: int = 32, ceil=None) -> dict:
    """The 1.3B decode step (24 layers, bf16 x, fp32 carried state h ~ N(0,1)) at each batch:
    one step of every layer captured in a HIP graph and replayed; per-kernel durations from an
    eager copy of 4 steps (events bound to each dispatch). At up to 16 rows the same step as one
    persistent kernel over the whole stack (mmf_stack_decode_step) is timed beside it."""
    from ternary_weight_matmul_amd import synth
    d, inner, L = synth.SHAPES["1.3B"]
    layers = device_layers(mmf, torch, d, inner, L, 3, dev)
    res = {}
    for b in batches:
        gen = torch.Generator(device=dev)
        gen.manual_seed(300 + b)
        hs = torch.randn((L, b, d), device=dev, generator=gen)
        xin = torch.randn((b, d), device=dev, generator=gen).to(torch.bfloat16)
        outs = [torch.empty_like(xin) for _ in range(2)]
        ws = torch.empty(mmf.layer_workspace_size(layers[0], b, 1), dtype=torch.uint8, device=dev)

        def step():
            y = xin
            for l in range(L):
                y = mmf.layer_decode_step(layers[l], y, hs[l], out=outs[l % 2], ws=ws)

        step()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        us = event_ms(torch, g.replay, steps, warmup=3) * 1000.0
        kt = KernelTable().add(timed_records(mmf, step, 4), "decode", 0.25)
        res[str(b)] = dict(us_per_layer=round(us / L, 2), us_per_token_step=round(us, 2),
                           layer_tokens_per_s=round(b * L / (us / 1e6), 1),
                           launches_per_layer=round(sum(e["launches"] for e in kt.k.values()) / L, 1),
                           roofline=with_ceiling(kt.roofline(us / 1000.0), ceil), kernels=kt.breakdown(4))
        if b <= 16:
            # the same step as one persistent kernel over all 24 layers (cooperative launches, eager)
            dec = mmf.StackDecoder(layers, [hs[l] for l in range(L)], b)
            sus = event_ms(torch, lambda: dec.step(xin, out=outs[0]), steps, warmup=3) * 1000.0
            res[str(b)]["stack_kernel"] = dict(us_per_layer=round(sus / L, 2), us_per_token_step=round(sus, 2),
                                               launches_per_token_step=2, expired_waits=mmf.stack_decode_expired())
            del dec
        del hs, xin, outs, ws, g
    del layers
    return dict(workload="1.3B decode step: 24 layers d=2048 inner=5632, bf16 x, fp32 state, HIP graph", by_batch=res)


def leg_c5(mmf, torch, dev, reps: int = 10, ceil=None, cpu: bool = True) -> dict:
    """The long-sequence scan stress at 1.3B width: x~ ~ N(0,1) and f = sigmoid(N(2,1)) fp32,
    16 x 32768 x 2048 (4 GiB each), chunked scan, h out of place; value = tokens/s (b*t per
    second). The oracle runs the sequential scan on a sample (one sequence, 256 channels)."""
    b, t, d = 16, 32768, 2048
    gen = torch.Generator(device=dev)
    gen.manual_seed(5)
    x = torch.randn((b, t, d), device=dev, generator=gen)
    f = torch.sigmoid(torch.randn((b, t, d), device=dev, generator=gen) + 2.0)
    h = torch.empty_like(x)

    def run():
        mmf.hgrn_scan_fwd(x, f, None, "chunk", out=h)

    ms = event_ms(torch, run, reps)
    kt = KernelTable().add(timed_records(mmf, run, reps), "scan", 1.0 / reps)
    res = dict(workload="HGRN scan stress: d=2048, B=16 x T=32768, fp32, chunked", value=round(b * t / (ms / 1000), 1),
               unit="tokens/s", ms=round(ms, 3), roofline=with_ceiling(kt.roofline(ms), ceil), kernels=kt.breakdown())
    if cpu:
        import numpy as np
        import oracle
        xs = x[0, :, :256].double().cpu().numpy()[None]
        fs = f[0, :, :256].double().cpu().numpy()[None]
        t0 = time.perf_counter()
        oracle.hgrn_scan(xs, fs)
        dt = time.perf_counter() - t0
        res["cpu_oracle"] = dict(value=round(t * 256 / d / dt, 1), unit="tokens/s (full-width equivalent)",
                                 cores=oracle.num_threads(), cpu=cpu_model(),
                                 sample="sequential scan of one sequence x 256 of 2048 channels (%.2f s), "
                                        "scaled to the full width" % dt)
        del xs, fs
    del x, f, h
    return res


def leg_hgrn2(mmf, torch, dev, reps: int = 5, ceil=None, cpu: bool = True) -> dict:
    """The expanded-state recurrence at 1.3B width, heads of 128: a 16 x 2048-token prefill
    (value = tokens/s; the chunked form on fp32 MFMA, with the step-wise form, bound by the fp32
    vector ALU, timed beside it) and a decode step at batch 16 (one token, the state read and
    written in place, HBM-bound). f = sigmoid(N(2,1)), i, o ~ N(0,1), the initial state ~ N(0,1).
    The oracle runs one (sequence, head) pair of the prefill."""
    b, t, d, e = 16, 2048, 2048, 128
    gen = torch.Generator(device=dev)
    gen.manual_seed(6)
    f = torch.sigmoid(torch.randn((b, t, d), device=dev, generator=gen) + 2.0)
    i = torch.randn((b, t, d), device=dev, generator=gen)
    o = torch.randn((b, t, d), device=dev, generator=gen)
    s0 = torch.randn((b, d // e, e, e), device=dev, generator=gen)
    s_last = torch.empty_like(s0)
    y = torch.empty_like(f)

    def run():
        mmf.hgrn2_scan_fwd(f, i, o, e, s0, out=y, s_last=s_last)

    ms = event_ms(torch, run, reps)
    kt = KernelTable().add(timed_records(mmf, run, reps), "prefill", 1.0 / reps)
    res = dict(workload="HGRN2 expanded-state recurrence: d=2048, heads of 128, B=16 x T=2048, fp32",
               value=round(b * t / (ms / 1000), 1), unit="tokens/s", ms=round(ms, 3),
               roofline=kt.roofline(ms), kernels=kt.breakdown())

    def run_steps():
        mmf.hgrn2_scan_fwd(f, i, o, e, s0, out=y, s_last=s_last, mode="recurrent")

    rms = event_ms(torch, run_steps, reps)
    kr = KernelTable().add(timed_records(mmf, run_steps, reps), "prefill", 1.0 / reps)
    res["prefill_step_wise"] = dict(ms=round(rms, 3), roofline=kr.roofline(rms))
    # decode: one token per sequence, the state updated in place
    f1, i1, o1 = f[:, :1].contiguous(), i[:, :1].contiguous(), o[:, :1].contiguous()
    st = s0.clone()
    y1 = torch.empty_like(f1)
    steps = 50

    def step():
        mmf.hgrn2_scan_fwd(f1, i1, o1, e, st, out=y1, s_last=st)

    sms = event_ms(torch, step, steps)
    kd = KernelTable().add(timed_records(mmf, step, steps), "decode", 1.0 / steps)
    res["decode_step"] = dict(workload="one token at B=16, state in place", us=round(sms * 1000, 2),
                              roofline=with_ceiling(kd.roofline(sms), ceil))
    if cpu:
        import oracle
        fs = f[0, :, :e].double().cpu().numpy()[None]
        is_ = i[0, :, :e].double().cpu().numpy()[None]
        os_ = o[0, :, :e].double().cpu().numpy()[None]
        s0s = s0[0, :1].double().cpu().numpy()[None]
        t0 = time.perf_counter()
        oracle.hgrn2_scan(fs, is_, os_, e, s0s)
        dt = time.perf_counter() - t0
        res["cpu_oracle"] = dict(value=round(t / (d // e) / dt, 1), unit="tokens/s (full-width equivalent)",
                                 cores=1, cpu=cpu_model(),
                                 sample="one sequence x one head of 16 (2048 tokens, %.2f s), scaled to the "
                                        "full width" % dt)
    del f, i, o, s0, s_last, y, st
    return res


def leg_gemv(mmf, torch, dev, ceil=None, reps: int = 10) -> dict:
    """Large FusedBitLinear products at 16 rows (bf16 in and out): the decode GEMV's streaming
    rate on 67 MB (16384 x 16384) and 268 MB (32768 x 32768) of packed ternary weights, from
    latent weights ~ N(0, 0.02) and x ~ N(0, 1). Roofline of the GEMV kernel itself (the row
    quantiser in front of it is timed too, apart); the packing of those weights is timed once."""
    out = {}
    for n, k in ((16384, 16384), (32768, 32768)):
        gen = torch.Generator(device=dev)
        gen.manual_seed(7)
        w = torch.randn((n, k), device=dev, generator=gen) * 0.02
        pl = mmf.ternary_pack(w)  # warm-up (and the weights used below)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        mmf.ternary_pack(w)
        b.record()
        torch.cuda.synchronize()
        pack_ms = a.elapsed_time(b)
        del w
        x = torch.randn((16, k), device=dev, generator=gen).to(torch.bfloat16)

        def run():
            mmf.bitlinear_fwd(x, pl)

        ms = event_ms(torch, run, reps)
        kt = KernelTable().add(timed_records(mmf, run, reps), "decode", 1.0 / reps)
        key = [kk for kk in kt.k if kk.startswith("tgemv")][0]
        # the packer reads the fp32 latent weights twice (mean |W|, then the codes) and writes 2 bits each
        pack_bytes = n * k * 8.25
        out["%dx%d" % (n, k)] = dict(weight_MB=round(n * k / 4 / 1e6, 1), us_per_call=round(ms * 1000, 2),
                                     roofline=with_ceiling(kt.roofline(ms, key), ceil),
                                     pack=dict(ms=round(pack_ms, 3), GBs=round(pack_bytes / (pack_ms / 1e3) / 1e9, 1),
                                               frac_hbm=round(pack_bytes / (pack_ms / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
                                               note="two passes over the fp32 weights: 8.25 B per weight"))
        del pl, x
        torch.cuda.empty_cache()
    return dict(workload="FusedBitLinear at 16 rows, bf16, packed ternary weights of 67 and 268 MB", shapes=out)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def run_only(args):
    """One leg alone (for profiling a config under rocprofv3): prints its JSON."""
    import torch
    import ternary_weight_matmul_amd as mmf
    mmf.load()
    dev = torch.device("cuda", 0)
    cpu = args.cpu_baseline != 0
    if args.only == "c1":
        res = leg_c1(mmf, torch, dev, cpu=cpu)
    elif args.only == "c2":
        res = leg_prefill(mmf, torch, dev, "370M", 8, 2048, 2, 5)
    elif args.only == "c4":
        res = leg_prefill(mmf, torch, dev, "2.7B", 4, 4096, 4, 3)
    elif args.only == "prefill_b8":
        res = leg_prefill(mmf, torch, dev, "1.3B", 8, 2048, 3, 3)
    elif args.only == "c3":
        res = leg_decode(mmf, torch, dev)
    elif args.only == "c5":
        res = leg_c5(mmf, torch, dev, cpu=cpu)
    elif args.only == "hgrn2":
        res = leg_hgrn2(mmf, torch, dev, cpu=cpu)
    elif args.only == "gemv":
        res = leg_gemv(mmf, torch, dev)
    elif args.only == "bwd":
        from ternary_weight_matmul_amd import synth
        d, inner, _ = synth.SHAPES["1.3B"]
        layer = device_layers(mmf, torch, d, inner, 1, 3, dev)[0]
        res = dict(scan_bwd=measure_scan_bwd(mmf, torch, 16, 2048, d, dev),
                   bitlinear_bwd=measure_bitlinear_bwd(mmf, torch, layer.o, 16 * 2048, dev),
                   bitlinear_bwd_gate=measure_bitlinear_bwd(mmf, torch, layer.gate, 16 * 2048, dev),
                   layer_bwd=measure_layer_bwd(mmf, torch, layer, 16, 2048, d, dev))
    else:
        res = hbm_ceilings(mmf, torch, dev)
        res["mfma"] = mfma_ceiling(mmf, torch, dev)
    print(json.dumps({"leg": args.only, **res}), flush=True)


def stored_trace_us(key: str):
    """(average duration in us, file) of kernel `key` from a rocprofv3 kernel-trace summary under
    profiles/ (lines "bench_kernel: <key>", "trace_avg_us: <us>", "sources: <digest>"), if one
    exists for the current sources of that kernel."""
    pdir = os.path.join(ROOT, "profiles")
    files = kernel_files(key)
    if not os.path.isdir(pdir) or not files:
        return None
    digest = source_digest(files)
    for name in sorted(os.listdir(pdir)):
        if not name.startswith("kernel_stats_"):
            continue
        cur = {}
        with open(os.path.join(pdir, name)) as f:
            for line in f:
                kk, _, vv = line.partition(":")
                kk = kk.strip()
                if kk == "bench_kernel":
                    cur = {"bench_kernel": vv.strip()}
                elif kk in ("trace_avg_us", "sources") and cur:
                    cur[kk] = vv.strip()
                    if cur.get("bench_kernel") == key and cur.get("sources") == digest and "trace_avg_us" in cur:
                        return float(cur["trace_avg_us"]), name
    return None


def main():
    args = parse()
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.vendor_int8_gemm:
        vendor_int8_gemm(args.shape, args.batch, args.prompt)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path; run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.only:
        run_only(args)
        return
    import numpy as np
    import torch
    import ternary_weight_matmul_amd as mmf
    from ternary_weight_matmul_amd import synth

    mmf.load()
    dev = torch.device("cuda", 0)
    d, inner, L = synth.SHAPES[args.shape]
    B, T, D = args.batch, args.prompt, args.decode
    seed = 3

    # ---- untimed preparation: weights ternarised + packed on the device, inputs resident in HBM
    t0 = time.time()
    layers = device_layers(mmf, torch, d, inner, L, seed, dev)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 10 + 1)
    x_prefill = torch.randn((B, T, d), device=dev, generator=gen).to(torch.bfloat16)
    x_decode = torch.randn((max(D, 1), B, d), device=dev, generator=gen).to(torch.bfloat16)
    bufs = [torch.empty_like(x_prefill) for _ in range(2)]
    hs = torch.zeros((L, B, d), dtype=torch.float32, device=dev)
    ws_p = torch.empty(mmf.layer_workspace_size(layers[0], B, T), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(mmf.layer_workspace_size(layers[0], B, 1), dtype=torch.uint8, device=dev)
    xin = torch.empty((B, d), dtype=torch.bfloat16, device=dev)
    douts = [torch.empty((B, d), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    torch.cuda.synchronize()
    prep_s = time.time() - t0

    def prefill():
        cur = x_prefill
        for l in range(L):
            out = bufs[l % 2]
            mmf.layer_fwd(layers[l], cur, None, out=out, h_last=hs[l], ws=ws_p)
            cur = out

    def decode_step():
        y = xin
        for l in range(L):
            y = mmf.layer_decode_step(layers[l], y, hs[l], out=douts[l % 2], ws=ws_d)

    graph = None
    if D > 0 and not args.no_graph:
        prefill()  # state for the capture warm-up
        xin.copy_(x_decode[0])
        decode_step()  # eager warm-up before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            decode_step()
        torch.cuda.synchronize()

    def decode():
        for s in range(D):
            xin.copy_(x_decode[s])
            if graph is not None:
                graph.replay()
            else:
                decode_step()

    for _ in range(args.warmup):
        prefill()
        decode()
    torch.cuda.synchronize()

    # ---- timed region: K steps; prefill kernels timed per dispatch on their stream
    mmf.timing_enable(True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        prefill()
        ev[i][1].record()
        decode()
        ev[i][2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t_start
    mmf.timing_enable(False)
    recs = mmf.timing_collect()
    prefill_ms = float(np.mean([a.elapsed_time(b) for a, b, _ in ev]))
    decode_ms = float(np.mean([b.elapsed_time(c) for _, b, c in ev]))

    # ---- decode kernels: the timed region replays them inside a HIP graph, where no event can
    # be bound to one kernel. The same decode steps are issued once more eagerly behind a queued
    # prefill (so the device never waits on the host between them), each kernel timed by events
    # bound to its own dispatch: its start and end, as a kernel trace records them.
    DM = min(4, D)
    drecs = []
    if DM:
        prefill()
        mmf.timing_enable(True)
        for s_ in range(DM):
            xin.copy_(x_decode[s_])
            decode_step()
        torch.cuda.synchronize()
        mmf.timing_enable(False)
        drecs = mmf.timing_collect()

    ms_per_step = elapsed * 1000.0 / args.steps
    tokens = B * (T + D)
    value = tokens * L / (ms_per_step / 1000.0)

    kt = KernelTable()
    kt.add(recs, "prefill", 1.0 / args.steps)
    if DM:
        kt.add(drecs, "decode", float(D) / DM)
    ex = args.extras != 0
    ceil = hbm_ceilings(mmf, torch, dev) if ex else None
    if ceil:
        ceil["mfma"] = mfma_ceiling(mmf, torch, dev)
    roof = with_ceiling(kt.roofline(ms_per_step), ceil)

    # ---- outside the timed region: every other config of the workload, the derivatives and
    # generation, each with its own roofline
    configs = None
    scan_bwd = bitlinear_bwd = layer_bwd = generate = None
    if ex:
        del bufs, ws_p
        torch.cuda.empty_cache()
        configs = {}
        configs["c1"] = leg_c1(mmf, torch, dev, cpu=args.cpu_baseline != 0)
        configs["c2"] = leg_prefill(mmf, torch, dev, "370M", 8, 2048, 2, 5, ceil)
        configs["c3"] = leg_decode(mmf, torch, dev, ceil=ceil)
        configs["c4"] = leg_prefill(mmf, torch, dev, "2.7B", 4, 4096, 4, 3, ceil)
        configs["prefill_1p3b_b8"] = leg_prefill(mmf, torch, dev, "1.3B", 8, 2048, 3, 3, ceil)
        torch.cuda.empty_cache()
        configs["c5"] = leg_c5(mmf, torch, dev, ceil=ceil, cpu=args.cpu_baseline != 0)
        torch.cuda.empty_cache()
        configs["hgrn2"] = leg_hgrn2(mmf, torch, dev, ceil=ceil, cpu=args.cpu_baseline != 0)
        torch.cuda.empty_cache()
        configs["gemv_stream"] = leg_gemv(mmf, torch, dev, ceil=ceil)
        torch.cuda.empty_cache()
        if T > 0:
            scan_bwd = measure_scan_bwd(mmf, torch, B, T, d, dev)
            bitlinear_bwd = measure_bitlinear_bwd(mmf, torch, layers[0].o, B * T, dev)
            layer_bwd = measure_layer_bwd(mmf, torch, layers[0], B, T, d, dev)
        if D:
            generate = [measure_generate(mmf, torch, layers, bb, d, dev, seed) for bb in (1, B)]

    cpu = None
    if args.cpu_baseline:
        cpu = cpu_baseline(d, inner, seed)

    line = {
        "metric": "HGRNBit layer tokens/s (prefill + decode), 1.3B shape; % HBM / int8 MFMA peak",
        "value": round(value, 1),
        "unit": "layer-tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 x ternary -> int32 contraction; bf16 activations; fp32 state",
        "data": "synthetic: x ~ N(0,1) bf16 and latent weights ~ N(0,0.02) drawn on the device (seeded), "
                "ternarised and packed on the device",
        "config": {
            "workload": "hgrnbit-%s-serve: %d layers d=%d inner=%d, prefill B=%d x T=%d, then %d decode steps" % (
                args.shape, L, d, inner, B, T, D),
            "layers": L, "d": d, "inner": inner, "batch": B, "prompt_tokens": T, "decode_steps": D,
            "decode_launch": "hip-graph" if graph is not None else "eager",
        },
        "roofline": roof,
        "cpu_baseline": cpu,
        "stack_tokens_per_s": round(tokens / (ms_per_step / 1000.0), 1),
        "prefill_ms": round(prefill_ms, 3),
        "decode_ms": round(decode_ms, 3),
        "prefill_layer_tokens_per_s": round(B * T * L / (prefill_ms / 1000), 1),
        "decode_layer_tokens_per_s": round(B * D * L / (decode_ms / 1000), 1) if D else None,
        "decode_us_per_token_step": round(decode_ms * 1000 / D, 2) if D else None,
        "decode_us_per_layer": round(decode_ms * 1000 / D / L, 2) if D else None,
        "decode_kernel_sum_us_per_token_step": round(kt.total_ms("decode") * 1000 / D, 2) if D else None,
        "prefill_contraction_roofline": contractions_with_ceiling(kt.contractions(), ceil),
        "hbm_ceiling": ceil,
        "configs": configs,
        "scan_bwd": scan_bwd,
        "bitlinear_bwd": bitlinear_bwd,
        "layer_bwd": layer_bwd,
        "generate": generate,
        "kernels": kt.breakdown(),
        "kernel_ms_per_step": round(kt.total_ms(), 3),
        "sources": source_digest(),
        "prep_s": round(prep_s, 1),
    }
    print(json.dumps(line), flush=True)


def measure_scan_bwd(mmf, torch, b: int, t: int, d: int, dev, launches: int = 10) -> dict:
    """The derivative of the recurrence (mmf_hgrn_scan_bwd, chunked) on seeded f, h, dh of the
    prefill's scan shape, timed per launch with HIP events on its stream."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(37)
    f = torch.sigmoid(torch.randn((b, t, d), device=dev, generator=gen) + 2.0)
    h = torch.randn((b, t, d), device=dev, generator=gen)
    dh = torch.randn((b, t, d), device=dev, generator=gen)
    dx, df = torch.empty_like(f), torch.empty_like(f)
    mmf.hgrn_scan_bwd(f, h, dh, None, None, "chunk", dx=dx, df=df)
    torch.cuda.synchronize()
    mmf.timing_enable(True)
    for _ in range(launches):
        mmf.hgrn_scan_bwd(f, h, dh, None, None, "chunk", dx=dx, df=df)
    torch.cuda.synchronize()
    mmf.timing_enable(False)
    recs = mmf.timing_collect()
    name = recs[0][0]
    avg_s = sum(r[4] for r in recs) / len(recs) / 1000.0
    _, nbytes = algorithmic(name, b * t, d, d)
    gbs = nbytes / avg_s / 1e9
    del f, h, dh, dx, df
    return dict(kernel="%s m=%d n=%d k=%d" % (name, b * t, d, d), shape="b=%d t=%d d=%d" % (b, t, d),
                avg_launch_us=round(avg_s * 1e6, 2), algorithmic_per_launch=nbytes, achieved=round(gbs, 1),
                peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4))


def measure_bitlinear_bwd(mmf, torch, lin, m: int, dev, launches: int = 5) -> dict:
    """The straight-through derivative of one FusedBitLinear (mmf_bitlinear_bwd: dx, dW and
    dgain, bf16 x and dy) at m rows, per kernel with HIP events: the two bf16 products against
    the dense bf16 MFMA peak, the rest against HBM."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(41)
    x = torch.randn((m, lin.k), device=dev, generator=gen).to(torch.bfloat16)
    dy = torch.randn((m, lin.n), device=dev, generator=gen).to(torch.bfloat16)
    mmf.bitlinear_bwd(x, lin, dy, want_dgain=True)
    torch.cuda.synchronize()
    mmf.timing_enable(True)
    for _ in range(launches):
        mmf.bitlinear_bwd(x, lin, dy, want_dgain=True)
    torch.cuda.synchronize()
    mmf.timing_enable(False)
    per = {}
    for name, mm, nn, kk, ms in mmf.timing_collect():
        e = per.setdefault(name, dict(m=mm, n=nn, k=kk, ms=0.0))
        e["ms"] += ms / launches
    total_ms = sum(e["ms"] for e in per.values())
    gemm_ms = sum(e["ms"] for k_, e in per.items() if k_.startswith("gemm_bf16"))
    flops = sum(2.0 * e["m"] * e["n"] * e["k"] for k_, e in per.items() if k_.startswith("gemm_bf16"))
    kernels = {k_: round(e["ms"] * 1000, 1) for k_, e in sorted(per.items(), key=lambda kv: -kv[1]["ms"])}
    del x, dy
    tf = flops / (gemm_ms / 1000) / 1e12
    return dict(shape="m=%d n=%d k=%d" % (m, lin.n, lin.k), us_per_call=round(total_ms * 1000, 1),
                kernels_us=kernels, gemm_achieved=round(tf, 1), peak=BF16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                gemm_frac=round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
                note="hand-written bf16 products (fp32 accumulation), operand layouts and RMSNorm derivative")


def measure_layer_bwd(mmf, torch, layer, b: int, t: int, d: int, dev, launches: int = 2) -> dict:
    """The block's derivative (mmf_layer_bwd: the forward recomputed, then every derivative, all
    weight and gain derivatives) on seeded bf16 x and dout of b x t tokens, timed with events."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(43)
    x = torch.randn((b, t, d), device=dev, generator=gen).to(torch.bfloat16)
    dout = torch.randn((b, t, d), device=dev, generator=gen).to(torch.bfloat16)
    res = mmf.layer_bwd(layer, x, dout, want_gains=True)
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(launches):
        res = mmf.layer_bwd(layer, x, dout, want_gains=True)
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / launches
    del x, dout, res
    return dict(shape="b=%d t=%d d=%d" % (b, t, d), ms_per_call=round(ms, 2),
                tokens_per_s=round(b * t / (ms / 1000), 1),
                note="forward recomputed inside; hand-written bf16 products of the derivative")


def measure_generate(mmf, torch, layers, b: int, d: int, dev, seed: int, vocab: int = 32000,
                     steps: int = 64) -> dict:
    """The token-to-token loop at batch b: embedding rows of a seeded bf16 table -> one decode
    step of every block -> greedy FusedBitLinear head over `vocab` tokens, whose tokens feed the
    next step on the device; one loop step captured in a HIP graph and replayed `steps` times."""
    L = len(layers)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 7919 + b)
    table = torch.randn((vocab, d), device=dev, generator=gen).to(torch.bfloat16)
    w_head = torch.randn((vocab, d), device=dev, generator=gen) * 0.02
    head = mmf.ternary_pack(w_head)
    del w_head
    ids = torch.randint(0, vocab, (b,), device=dev, dtype=torch.int32, generator=gen)
    hs = torch.randn((L, b, d), device=dev, generator=gen)
    x = torch.empty((b, d), dtype=torch.bfloat16, device=dev)
    outs = [torch.empty_like(x) for _ in range(2)]
    ws = torch.empty(mmf.layer_workspace_size(layers[0], b, 1), dtype=torch.uint8, device=dev)

    def step():
        mmf.embed(ids, table, out=x)
        y = x
        for l in range(L):
            y = mmf.layer_decode_step(layers[l], y, hs[l], out=outs[l % 2], ws=ws)
        mmf.greedy_head(y, head, tokens=ids)

    step()
    torch.cuda.synchronize()
    mmf.timing_enable(True)
    y = outs[(L - 1) % 2]
    for _ in range(4):
        mmf.greedy_head(y, head, tokens=ids)
    torch.cuda.synchronize()
    mmf.timing_enable(False)
    head_us = sum(r[4] for r in mmf.timing_collect()) * 1000.0 / 4
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    us = (time.perf_counter() - t0) * 1e6 / steps
    return dict(batch=b, vocab=vocab, layers=L, us_per_token_step=round(us, 1),
                tokens_per_s=round(b / (us / 1e6), 1), head_us_eager=round(head_us, 1),
                note="embed + %d decode blocks + greedy ternary head per step, HIP graph, tokens stay on the device" % L)


def cpu_baseline(d: int, inner: int, seed: int) -> dict:
    """The oracle (plain C + numpy fp64, OpenMP over independent outputs) on a bounded sample:
    one layer of the same shape, a 1024-token prefill of one sequence plus 16 decode steps at
    batch 16 continuing from random states."""
    import numpy as np
    import oracle
    from ternary_weight_matmul_amd import synth

    lat = synth.latent_weights(d, inner, synth.layer_seed(seed, 0))
    Lo = oracle.make_layer(lat)
    del lat
    T0, S0, B0 = 1024, 16, 16
    x = synth.activations((1, T0, d), seed * 10 + 1, "bf16")
    xs = synth.activations((S0, B0, d), seed * 10 + 2, "bf16")
    h = synth.rng(seed * 10 + 3).standard_normal((B0, d))
    t0 = time.perf_counter()
    oracle.layer_forward(Lo, x)
    for s_ in range(S0):
        h = oracle.layer_decode_step(Lo, xs[s_], h)["h"]
    dt = time.perf_counter() - t0
    tokens = T0 + S0 * B0
    return {"value": round(tokens / dt, 2), "unit": "layer-tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle", "cpu": cpu_model(),
            "sample": "1 layer at the same shape: prefill of 1x%d tokens + %d decode steps at batch %d "
                      "(%d layer-tokens, %.1f s)" % (T0, S0, B0, tokens, dt)}


if __name__ == "__main__":
    main()
