#!/usr/bin/env python3
"""HGRNBit layer throughput on one MI355X: prefill + decode at the 1.3B shape.

One step is one serving pass over one batch of seeded synthetic input through
a 24-layer HGRNBit stack (d=2048, MLP inner 5632, random ternarised weights):
  1. prefill: B sequences of T prompt tokens through every layer (chunked scan);
  2. decode: D tokens per sequence, one layer step at a time, each continuing
     from the state the prefill left in that layer.
value = layer-tokens/s = B*(T+D)*L / step time (metric "HGRNBit layer tokens/s").

Also printed in the same JSON line:
  roofline     -- the dominant kernel (largest share of the step's kernel time,
                  measured with HIP events on the launch stream over the timed
                  steps) against its roof: int8 MFMA peak for the prefill
                  contraction, HBM for the decode weight stream;
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
    return ap.parse_args()


def algorithmic(kernel: str, m: int, n: int, k: int):
    """(ops, bytes) one launch must do: ops = 2*m*n*k for a contraction; bytes = packed
    weights (n*k/4) + int8 codes (m*k) + per-row scale/sum (8m) + outputs (4 bytes per output element)."""
    if kernel.startswith("tgemm") or kernel.startswith("tgemv"):
        ops = 2.0 * m * n * k
        out_elems = {"gates": 3 * (n // 3), "gates_step": 3 * (n // 3), "glu": n // 2}.get(
            kernel.split("<")[1].split(">")[0].split(",")[0], n)
        nbytes = n * k / 4.0 + m * k + 8.0 * m + 4.0 * m * out_elems
        return ops, nbytes
    return 0.0, 0.0


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path; run with --gpus 1", file=sys.stderr)
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

    # ---- timed region: K steps; prefill kernels bracketed by HIP events
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

    # decode kernels run inside the graph: time one eager instrumented decode step after the timed region
    mmf.timing_enable(True)
    xin.copy_(x_decode[0])
    decode_step()
    torch.cuda.synchronize()
    mmf.timing_enable(False)
    drecs = mmf.timing_collect()

    ms_per_step = elapsed * 1000.0 / args.steps
    tokens = B * (T + D)
    value = tokens * L / (ms_per_step / 1000.0)

    # ---- per-kernel summary
    per = {}
    for name, m, n, k, ms in recs:
        e = per.setdefault(name, dict(launches=0, ms=0.0, ops=0.0, bytes=0.0, phase="prefill"))
        ops, nb = algorithmic(name, m, n, k)
        e["launches"] += 1
        e["ms"] += ms
        e["ops"] += ops
        e["bytes"] += nb
    dper = {}
    for name, m, n, k, ms in drecs:
        e = dper.setdefault(name, dict(launches=0, ms=0.0, ops=0.0, bytes=0.0, phase="decode"))
        ops, nb = algorithmic(name, m, n, k)
        e["launches"] += 1
        e["ms"] += ms
        e["ops"] += ops
        e["bytes"] += nb
    # decode totals over the timed region: one instrumented step scaled by D steps and K repetitions
    for e in dper.values():
        for key in ("launches", "ms", "ops", "bytes"):
            e[key] *= D * args.steps
    kernels = {}
    for src in (per, dper):
        for name, e in src.items():
            key = name if name not in kernels else name + "@" + e["phase"]
            kernels[key] = e
    dom_name, dom = max(kernels.items(), key=lambda kv: kv[1]["ms"])
    avg_ms = dom["ms"] / dom["launches"]
    if dom_name.startswith("tgemm"):
        achieved = dom["ops"] / dom["launches"] / (avg_ms / 1000.0) / 1e12
        roof = dict(bound="mfma", achieved=round(achieved, 2), peak=INT8_MFMA_PEAK_TOPS, unit="TFLOP/s")
    else:
        achieved = dom["bytes"] / dom["launches"] / (avg_ms / 1000.0) / 1e9
        roof = dict(bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s")
    roof["frac"] = round(roof["achieved"] / roof["peak"], 4)
    roof["traffic"] = None
    roof["kernel"] = dom_name
    roof["avg_launch_us"] = round(avg_ms * 1000.0, 2)
    roof["share_of_kernel_time"] = round(dom["ms"] / sum(e["ms"] for e in kernels.values()), 3)

    breakdown = {}
    for name, e in sorted(kernels.items(), key=lambda kv: -kv[1]["ms"]):
        avg = e["ms"] / e["launches"]
        row = dict(launches=int(e["launches"]), avg_us=round(avg * 1000, 2), total_ms=round(e["ms"] / args.steps, 3))
        if e["ops"]:
            row["tops"] = round(e["ops"] / e["launches"] / (avg / 1000) / 1e12, 1)
            row["gbs"] = round(e["bytes"] / e["launches"] / (avg / 1000) / 1e9, 1)
        breakdown[name] = row

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
        "dtype": "int8xternary->int32 contraction; bf16 activations; fp32 state",
        "data": "synthetic: seeded x~N(0,1) bf16, latent weights~N(0,0.02) ternarised on device",
        "config": {
            "workload": "hgrnbit-%s-serve: %d layers d=%d inner=%d, prefill B=%d x T=%d, then %d decode steps" % (
                args.shape, L, d, inner, B, T, D),
            "layers": L, "d": d, "inner": inner, "batch": B, "prompt_tokens": T, "decode_steps": D,
            "decode_launch": "hip-graph" if graph is not None else "eager",
        },
        "prefill_ms": round(prefill_ms, 3),
        "decode_ms": round(decode_ms, 3),
        "prefill_layer_tokens_per_s": round(B * T * L / (prefill_ms / 1000), 1),
        "decode_layer_tokens_per_s": round(B * D * L / (decode_ms / 1000), 1) if D else None,
        "decode_us_per_token_step": round(decode_ms * 1000 / D, 2) if D else None,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": breakdown,
        "prep_s": round(prep_s, 1),
    }
    print(json.dumps(line), flush=True)


def cpu_baseline(d: int, inner: int, seed: int) -> dict:
    """The oracle (plain C + numpy fp64, OpenMP over independent outputs) on a bounded sample:
    one layer of the same shape, a 256-token prefill of one sequence plus 4 decode steps at batch 16."""
    import numpy as np
    import oracle
    from ternary_weight_matmul_amd import synth

    lat = synth.latent_weights(d, inner, synth.layer_seed(seed, 0))
    Lo = oracle.make_layer(lat)
    del lat
    x = synth.activations((1, 256, d), seed * 10 + 1, "bf16")
    xs = synth.activations((4, 16, d), seed * 10 + 2, "bf16")
    t0 = time.perf_counter()
    r = oracle.layer_forward(Lo, x)
    h = np.zeros((16, d))
    for s in range(4):
        h = oracle.layer_decode_step(Lo, xs[s], h)["h"]
    dt = time.perf_counter() - t0
    tokens = 256 + 4 * 16
    return {"value": round(tokens / dt, 2), "unit": "layer-tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "1 layer at the same shape: prefill of 1x256 tokens + 4 decode steps at batch 16 (%d layer-tokens, %.1f s)" % (tokens, dt)}


if __name__ == "__main__":
    main()
