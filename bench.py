"""Benchmark of the EXL3 trellis linear layer on one MI355X.

Headline workload: the decode-phase merged gate_up projection (IC=4096; gate OC=14336 at K=2 and up
OC=14336 at K=3 written into column slices of one bf16 [M, 28672] output), M=1.  One step = one call
of the whole layer (activation pre-pass, both shards' trellis decode + contraction, split-K reduce,
output Hadamard and scales).  The metric is GB/s of trellis words (the method's algorithmic bytes,
IC*OC*K/8 per shard).  Weights rotate over 16 seeded copies (587 MB) so the 256 MiB Infinity Cache
cannot serve them.  Steps are captured once in a HIP graph and replayed between events.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EXL3 linear GB/s (trellis bytes) at M=1 & TFLOP/s at M=8192; % roofline"
HBM_PEAK_GBS = 8000.0
COPIES = 16


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--extra-m", default="2,4,8", help="additional decode M values reported under 'extra'")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=8192 prefill measurements")
    return ap.parse_args()


def build_gate_up(torch, dev, synth, copies):
    cfg = synth.DECODE_GATE_UP
    IC = cfg["IC"]
    rng = np.random.default_rng(1001)
    s_in = torch.from_numpy(synth.random_signs(rng, IC)).to(dev)
    rin = torch.from_numpy(synth.random_scales(rng, IC)).to(dev)
    sets = []
    for r in range(copies):
        rr = np.random.default_rng(5000 + r)
        shards, col = [], 0
        for OC, K in ((cfg["OC_gate"], cfg["K_gate"]), (cfg["OC_up"], cfg["K_up"])):
            s = synth.shard(rr, IC, OC, K)
            shards.append(dict(code=torch.from_numpy(s["code"]).to(dev), K=K, col0=col, s_in=s_in, rin=rin,
                               rout=torch.from_numpy(s["rout"]).to(dev), s_out=torch.from_numpy(s["s_out"]).to(dev)))
            col += OC
        sets.append(shards)
    trellis_bytes = sum(IC * s["code"].shape[1] * 16 * s["K"] // 8 for s in sets[0])
    return IC, col, sets, trellis_bytes


def time_decode(torch, exl3, dev, x, out, sets, steps, warmup):
    """Capture `warmup` and `steps` rotated calls in two graphs; return seconds per step."""
    M, IC = x.shape
    ws = exl3.alloc_workspace(max(exl3.linear_multi_workspace_bytes(M, IC, s) for s in sets), dev)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for s in sets:
            exl3.linear_multi_into(out, x, s, ws=ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for n in (warmup, steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                exl3.linear_multi_into(out, x, sets[i % len(sets)], ws=ws)
        graphs.append(g)
    torch.cuda.synchronize()
    graphs[0].replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record()
    graphs[1].replay()
    t1.record()
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / 1e3 / steps


def time_prefill(torch, exl3, synth, dev, reps=5):
    """M=8192 prefill projections: gate_up (IC=5120 -> 2 x 17408, K=2 | K=3) and down (17408 -> 5120, K=3).
    Returns {name: (seconds per call, FLOP per call)}; FLOP = 2*M*IC*OC (decode and transforms not counted)."""
    p = synth.PREFILL
    M = p["M"]
    res = {}
    rng = np.random.default_rng(4242)
    gu, dn = p["gate_up"], p["down"]
    for name, IC, shards in (("gate_up", gu["IC"], [(gu["OC"], gu["K_gate"]), (gu["OC"], gu["K_up"])]),
                             ("down", dn["IC"], [(dn["OC"], dn["K"])])):
        _, xb = synth.random_activations(rng, M, IC)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        s_in = torch.from_numpy(synth.random_signs(rng, IC)).to(dev)
        rin = torch.from_numpy(synth.random_scales(rng, IC)).to(dev)
        sh, col = [], 0
        for OC, K in shards:
            d = synth.shard(rng, IC, OC, K)
            sh.append(dict(code=torch.from_numpy(d["code"]).to(dev), K=K, col0=col, s_in=s_in, rin=rin,
                           rout=torch.from_numpy(d["rout"]).to(dev), s_out=torch.from_numpy(d["s_out"]).to(dev)))
            col += OC
        out = torch.empty((M, col), dtype=torch.bfloat16, device=dev)
        ws = exl3.alloc_workspace(exl3.linear_multi_workspace_bytes(M, IC, sh), dev)
        exl3.linear_multi_into(out, x, sh, ws=ws)
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        for _ in range(reps):
            exl3.linear_multi_into(out, x, sh, ws=ws)
        t1.record()
        torch.cuda.synchronize()
        sec = t0.elapsed_time(t1) / 1e3 / reps
        res[name] = (sec, 2.0 * M * IC * col)
        print(f"# prefill {name} M={M}: {sec * 1e3:.3f} ms/call, {res[name][1] / sec / 1e12:.1f} TFLOP/s",
              file=sys.stderr, flush=True)
        del x, out, ws, sh
    return res


def cpu_baseline(synth, O):
    """The fp64 oracle on one M=1 step of the same workload (both shards), single-threaded."""
    from threadpoolctl import threadpool_limits
    cfg = synth.DECODE_GATE_UP
    case = synth.merged_case(1001, 1, cfg["IC"], [(cfg["OC_gate"], cfg["K_gate"]), (cfg["OC_up"], cfg["K_up"])])
    with threadpool_limits(limits=1):
        t = time.perf_counter()
        for s in case["shards"]:
            O.linear(case["x"], s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"])
        dt = time.perf_counter() - t
    nbytes = sum(cfg["IC"] * s["OC"] * s["K"] // 8 for s in case["shards"])
    return dict(value=round(nbytes / dt / 1e9, 4), unit="GB/s", cores=1, kind="oracle",
                sample="one full M=1 step of the decode gate_up workload (both shards, fp64 numpy, 1 thread), "
                       f"{dt:.1f} s")


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (--gpus {a.gpus} requested); "
              "the multi-GPU sharding is described in DESIGN.md", file=sys.stderr)
        sys.exit(2)
    import torch
    from moe_exl3_pre_amd import exl3, synth
    dev = torch.device("cuda", 0)
    exl3.lib()

    IC, ldo, sets, trellis_bytes = build_gate_up(torch, dev, synth, COPIES)
    rng = np.random.default_rng(77)
    results = {}
    for M in [1] + [int(m) for m in a.extra_m.split(",") if m]:
        _, xb = synth.random_activations(rng, M, IC)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        out = torch.empty((M, ldo), dtype=torch.bfloat16, device=dev)
        sec = time_decode(torch, exl3, dev, x, out, sets, a.steps if M == 1 else max(a.steps // 4, COPIES),
                          a.warmup if M == 1 else COPIES)
        results[M] = sec
        print(f"# decode gate_up M={M}: {sec * 1e6:.2f} us/step, {trellis_bytes / sec / 1e9:.1f} GB/s trellis",
              file=sys.stderr, flush=True)

    prefill = {} if a.no_prefill else time_prefill(torch, exl3, synth, dev)

    sec = results[1]
    gbs = trellis_bytes / sec / 1e9
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "decode gate_up: IC=4096, gate OC=14336 K=2 | up OC=14336 K=3, M=1, "
                               f"{COPIES} rotated weight copies", "M": 1, "IC": IC, "OC": [14336, 14336], "K": [2, 3],
                   "trellis_bytes_per_step": trellis_bytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "whole step (pre-pass + both shards' decode-phase kernels)"},
        "extra": {f"decode_M{M}": {"us_per_step": round(s * 1e6, 3), "trellis_GBps": round(trellis_bytes / s / 1e9, 1)}
                  for M, s in results.items()},
    }
    for name, (s, flop) in prefill.items():
        line["extra"][f"prefill_{name}_M8192"] = {"ms_per_call": round(s * 1e3, 4), "TFLOPs": round(flop / s / 1e12, 1),
                                                  "frac_of_fp16_peak": round(flop / s / 2.5e15, 4)}
    if not a.no_cpu:
        from oracle import exl3_oracle as O
        line["cpu_baseline"] = cpu_baseline(synth, O)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
