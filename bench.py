#!/usr/bin/env python3
"""HGRNBit layer throughput on one MI355X: prefill + decode at the 1.3B shape.

One step is one serving pass over one batch of seeded synthetic input through
a 24-layer HGRNBit stack (d=2048, MLP inner 5632, random ternarised weights):
  1. prefill: B sequences of T prompt tokens through every layer (chunked scan);
  2. decode: D tokens per sequence, one layer step at a time, each continuing
     from the state the prefill left in that layer.
value = layer-tokens/s = B*(T+D)*L / step time (metric "HGRNBit layer tokens/s").

Also printed in the same JSON line:
  roofline     -- the dominant kernel at its shape (largest share of the step
                  time) against its roof: int8 MFMA peak for a prefill
                  contraction, HBM for everything else. Prefill kernels are
                  timed with HIP events on their stream inside the timed steps;
                  decode kernels, which run inside a HIP graph there, are timed
                  the same way on an eager copy of the decode steps queued
                  behind a prefill;
  cpu_baseline -- the CPU oracle on a bounded sample of the same workload.
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
                    help="0 skips the figures measured outside the timed steps (other batches, B=8 prefill, "
                         "derivatives, generation)")
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
        gates: f, x~ (fp32) and g (bf16) written = 10 B; gates_step: h read and written
        (fp32) and g written (bf16) = 10 B; glu: z (bf16) = 2 B; resid: residual read and
        sum written, one fp32 and one bf16 = 6 B; linear: 4 B.
    tgemv_row<epi,T> (a contraction that quantises its own input rows): as a contraction, with
      the rows read once in type T (m k sizeof T) in place of the codes, scale and code sum;
      tgemv_row<resid,gnorm,T>: h (fp32) and g (T) per element and g_norm's gain (fp32) per k.
    norm_quant<T> (m rows of k): x read (sizeof T) + codes written (1 B) per element, 8 B per row.
    gnorm_quant<T>: h (fp32) and g (sizeof T) read + codes written per element, 8 B per row.
    scan (m = b t, k = d): f and x~ read, h written, 12 B per element.
    scan_bwd (m = b t, k = d): dh, f and h read, dx and df written, 20 B per element.
    decode_step_xcd (m = b, n = d, k = inner; one whole decode step of a block): ops =
      2 b (4 d^2 + 3 d inner); bytes = all packed weights (4 d^2 + 3 d inner) / 4 + x read
      and out written (activation dtype) + h read and written (fp32) per row element.
    """
    base, args = _kind(kernel)
    if base == "decode_step_xcd":
        wts = 4.0 * n * n + 3.0 * n * k
        return 2.0 * m * wts, wts / 4.0 + m * n * (2.0 * ACT_BYTES + 8.0)
    if base in ("tgemm", "tgemm_dma", "tgemv", "tgemv_row"):
        epi = args[0]
        na = 3 if "split_a" in args else 1
        ng = {"gates": 3, "gates_step": 3, "glu": 2}.get(epi, 1)
        per_c = {"gates": 10, "gates_step": 10, "glu": 2, "resid": 4 + ACT_BYTES, "linear": 4}[epi]
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
    "tgemv_q": ["k_gemv_q.hip", "row_quant.hpp", "epilogue.hpp"] + _COMMON,
    "decode_step_xcd": ["k_decode.hip", "row_quant.hpp", "epilogue.hpp"] + _COMMON,
    "norm_quant": ["k_quant.hip", "row_quant.hpp"] + _COMMON,
    "gnorm_quant": ["k_quant.hip", "row_quant.hpp"] + _COMMON,
    "scan": ["k_scan.hip"] + _COMMON,
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
    layers = []
    for l in range(L):
        lat = synth.latent_weights(d, inner, synth.layer_seed(seed, l))
        layers.append(mmf.LayerParams.pack({k: torch.from_numpy(v).to(dev) for k, v in lat.items()}))
        del lat
    x_prefill = torch.from_numpy(synth.activations((B, T, d), seed * 10 + 1, "bf16")).to(dev).to(torch.bfloat16)
    x_decode = torch.from_numpy(synth.activations((max(D, 1), B, d), seed * 10 + 2, "bf16")).to(dev).to(torch.bfloat16)
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

    def step():
        prefill()
        decode()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K steps; prefill kernels bracketed by HIP events on their stream
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
    # bracket a single kernel. The same decode steps are issued once more eagerly, with the
    # per-launch events, behind a queued prefill so that the device never waits on the host
    # between them; their event-measured durations stand for the graph's (the sum is reported
    # next to the graph's own time per step as a check).
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

    # ---- per-kernel totals per step, keyed by variant and shape
    kernels = {}

    def add(src, phase, scale):
        for name, m, n, k, ms in src:
            key = "%s m=%d n=%d k=%d" % (name, m, n, k)
            e = kernels.setdefault(key, dict(name=name, m=m, n=n, k=k, phase=phase, launches=0.0, ms=0.0))
            e["launches"] += scale
            e["ms"] += ms * scale

    add(recs, "prefill", 1.0 / args.steps)
    if DM:
        add(drecs, "decode", float(D) / DM)
    for e in kernels.values():
        e["avg_ms"] = e["ms"] / e["launches"]
        e["ops"], e["bytes"] = algorithmic(e["name"], e["m"], e["n"], e["k"])
    total_kernel_ms = sum(e["ms"] for e in kernels.values())
    dom_key, dom = max(kernels.items(), key=lambda kv: kv[1]["ms"])
    avg_s = dom["avg_ms"] / 1000.0
    if dom["name"].startswith("tgemm"):
        achieved = dom["ops"] / avg_s / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=INT8_MFMA_PEAK_TOPS, unit="TFLOP/s")
    else:
        achieved = dom["bytes"] / avg_s / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = stored_traffic(dom_key)
    roof["kernel"] = dom_key
    roof["phase"] = dom["phase"]
    roof["avg_launch_us"] = round(dom["avg_ms"] * 1000.0, 2)
    roof["algorithmic_per_launch"] = dom["ops"] if roof["bound"] == "mfma" else dom["bytes"]
    roof["share_of_step"] = round(dom["ms"] / ms_per_step, 3)

    breakdown = {}
    for key, e in sorted(kernels.items(), key=lambda kv: -kv[1]["ms"]):
        row = dict(phase=e["phase"], launches_per_step=round(e["launches"], 1), avg_us=round(e["avg_ms"] * 1000, 2),
                   ms_per_step=round(e["ms"], 3))
        t = e["avg_ms"] / 1000.0
        if e["ops"]:
            row["int8_tops"] = round(e["ops"] / t / 1e12, 1)
            row["frac_mfma"] = round(e["ops"] / t / 1e12 / INT8_MFMA_PEAK_TOPS, 4)
        row["gbs"] = round(e["bytes"] / t / 1e9, 1)
        row["frac_hbm"] = round(e["bytes"] / t / 1e9 / HBM_PEAK_GBS, 4)
        breakdown[key] = row

    # the best prefill contraction against the MFMA roof, for reference next to the dominant kernel
    pre = [e for e in kernels.values() if e["phase"] == "prefill" and e["ops"]]
    prefill_gemm = None
    if pre:
        ops = sum(e["ops"] * e["launches"] for e in pre)
        ms = sum(e["ms"] for e in pre)
        prefill_gemm = dict(achieved=round(ops / (ms / 1000) / 1e12, 1), peak=INT8_MFMA_PEAK_TOPS, unit="TFLOP/s",
                            frac=round(ops / (ms / 1000) / 1e12 / INT8_MFMA_PEAK_TOPS, 4),
                            note="all prefill contractions together, int8 ops over their event-measured time")

    # ---- outside the timed region: the scan's derivative at the prefill's scan shape, and the
    # decode step at the other batch sizes of the 1.3B decode workload (graph-replayed)
    ex = args.extras != 0
    scan_bwd = measure_scan_bwd(mmf, torch, B, T, d, dev) if ex and T > 0 else None
    bitlinear_bwd = measure_bitlinear_bwd(mmf, torch, layers[0].o, B * T, dev) if ex and T > 0 else None
    layer_bwd = measure_layer_bwd(mmf, torch, layers[0], B, T, d, dev) if ex and T > 0 else None
    by_batch = {str(B): round(decode_ms * 1000 / D / L, 2)} if D else {}
    if ex and D and graph is not None:
        for bb in (1, 64):
            if bb != B:
                by_batch[str(bb)] = round(decode_us_per_layer(mmf, torch, layers, bb, d, dev, seed), 2)
    by_batch = dict(sorted(by_batch.items(), key=lambda kv: int(kv[0])))
    prefill_b8 = measure_prefill(mmf, torch, layers, 8, T, d, dev, seed) if ex and T > 0 and B != 8 else None
    generate = [measure_generate(mmf, torch, layers, bb, d, dev, seed) for bb in (1, B)] if ex and D else None

    cpu = None
    if args.cpu_baseline:
        cpu = cpu_baseline(d, inner, seed)

    dsum = sum(e["ms"] for e in kernels.values() if e["phase"] == "decode")
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
        "data": "synthetic: seeded x~N(0,1) bf16, latent weights~N(0,0.02) ternarised on device",
        "config": {
            "workload": "hgrnbit-%s-serve: %d layers d=%d inner=%d, prefill B=%d x T=%d, then %d decode steps" % (
                args.shape, L, d, inner, B, T, D),
            "layers": L, "d": d, "inner": inner, "batch": B, "prompt_tokens": T, "decode_steps": D,
            "decode_launch": "hip-graph" if graph is not None else "eager",
        },
        "stack_tokens_per_s": round(tokens / (ms_per_step / 1000.0), 1),
        "prefill_ms": round(prefill_ms, 3),
        "decode_ms": round(decode_ms, 3),
        "prefill_layer_tokens_per_s": round(B * T * L / (prefill_ms / 1000), 1),
        "decode_layer_tokens_per_s": round(B * D * L / (decode_ms / 1000), 1) if D else None,
        "decode_us_per_token_step": round(decode_ms * 1000 / D, 2) if D else None,
        "decode_kernel_sum_us_per_token_step": round(dsum * 1000 / D, 2) if D else None,
        "roofline": roof,
        "prefill_contraction_roofline": prefill_gemm,
        "decode_us_per_layer_by_batch": by_batch,
        "prefill_b8": prefill_b8,
        "scan_bwd": scan_bwd,
        "bitlinear_bwd": bitlinear_bwd,
        "layer_bwd": layer_bwd,
        "generate": generate,
        "cpu_baseline": cpu,
        "kernels": breakdown,
        "kernel_ms_per_step": round(total_kernel_ms, 3),
        "sources": source_digest(),
        "prep_s": round(prep_s, 1),
    }
    print(json.dumps(line), flush=True)


def measure_prefill(mmf, torch, layers, b: int, t: int, d: int, dev, seed: int, reps: int = 3) -> dict:
    """The whole-stack prefill alone at batch b (the 1.3B prefill read at b = 8, t = 2048), seeded
    bf16 input, timed with events over `reps` runs after one warm-up."""
    from ternary_weight_matmul_amd import synth
    L = len(layers)
    x = torch.from_numpy(synth.activations((b, t, d), seed * 10 + 5, "bf16")).to(dev).to(torch.bfloat16)
    bufs = [torch.empty_like(x) for _ in range(2)]
    hs = torch.empty((L, b, d), dtype=torch.float32, device=dev)
    ws = torch.empty(mmf.layer_workspace_size(layers[0], b, t), dtype=torch.uint8, device=dev)

    def run():
        cur = x
        for l in range(L):
            mmf.layer_fwd(layers[l], cur, None, out=bufs[l % 2], h_last=hs[l], ws=ws)
            cur = bufs[l % 2]

    run()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record()
    for _ in range(reps):
        run()
    ev[1].record()
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[1]) / reps
    del x, bufs, hs, ws
    return dict(batch=b, prompt_tokens=t, ms=round(ms, 3), layer_tokens_per_s=round(b * t * L / (ms / 1000), 1),
                stack_tokens_per_s=round(b * t / (ms / 1000), 1))


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
                note="products through rocBLAS (bf16, fp32 accumulation); the rest hand-written")


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
                note="forward recomputed inside; products of the derivative through rocBLAS (bf16)")


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


def decode_us_per_layer(mmf, torch, layers, b: int, d: int, dev, seed: int, steps: int = 32) -> float:
    """One decode step of every layer at batch b, captured in a HIP graph and replayed `steps`
    times from a seeded state; microseconds per layer."""
    L = len(layers)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed * 100 + b)
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
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / steps / L


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
            "kind": "oracle",
            "sample": "1 layer at the same shape: prefill of 1x%d tokens + %d decode steps at batch %d "
                      "(%d layer-tokens, %.1f s)" % (T0, S0, B0, tokens, dt)}


if __name__ == "__main__":
    main()
