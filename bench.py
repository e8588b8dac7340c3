"""Benchmark of the EXL3 trellis linear layer on one MI355X.

Headline workload: the decode-phase merged gate_up projection (IC=4096; gate OC=14336 at K=2 and up
OC=14336 at K=3 written into column slices of one bf16 [M, 28672] output), M=1.  One step = one call
of the whole layer (activation pre-pass, both shards' trellis decode + contraction, split-K reduce,
output Hadamard and scales), which is one kernel launch.  The metric is GB/s of trellis words (the
method's algorithmic bytes, IC*OC*K/8 per shard).  Weights rotate over 16 seeded copies (587 MB) so the
256 MiB Infinity Cache cannot serve them.  Steps are captured once in a HIP graph and replayed between
events recorded on the stream the kernels run on.

Also reported (under "extra"): decode M = 2, 4, 8; prefill M=8192 gate_up and down (TFLOP/s); the MoE
expert bank (T=256, E=128, top-8, H=2048, I=768; 3 rotated banks; also T=4096 in TFLOP/s); the dense MLP block of one decoder
layer (5120 -> 2 x 17408 -> 5120) at M = 1 and 8; the int8 embedding gather (T = 256 and 8192 ids over a
248,320 x 5120 table) and the same table as the output head (M = 1 and 16; GB/s of bytes moved).

Every timing is the median, p10 and p90 over at least 20 timed replays (graphs of captured calls, or eager
calls for the prefill projections) between events on the launching stream; the headline value is the mean
over exactly --steps calls.  Measured peaks (a 4 GiB streaming read; back-to-back f16 and i8 MFMAs) are
reported beside the published ones as secondary denominators.  The CPU baseline is the fp64 oracle on the
same step, on one thread and on all usable cores (with the host's CPU count and model).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-prefill] [--no-moe] [--no-mlp]
                    [--no-embed]
    python bench.py --pmc-ref ...     # eager launches plus a 1 GiB copy, for counter runs
    python bench.py --pmc-moe ...     # eager MoE bank calls (T=256, T=4096) plus 1 GiB copies, for counter runs
    python bench.py --pmc-int8        # the same for the int8 embedding gather and output head
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "EXL3 linear GB/s (trellis bytes) at M=1 & TFLOP/s at M=8192; % roofline"
HBM_PEAK_GBS = 8000.0
F16_PEAK_TFLOPS = 2500.0
I8_PEAK_TOPS = 5000.0
COPIES = 16
MOE_COPIES = 3
DECODE_KERNEL = "exl3::decode_kernel"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_gate_up_m1.md")
# sources whose change invalidates the stored counter readings of the decode kernel
TRAFFIC_SOURCES = ["moe_exl3_pre_amd/csrc/k_decode.hip", "moe_exl3_pre_amd/csrc/exl3_device.hpp",
                   "moe_exl3_pre_amd/csrc/exl3_internal.hpp", "moe_exl3_pre_amd/csrc/k_silu.hpp"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=480)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--extra-m", default="2,4,8", help="additional decode M values reported under 'extra'")
    ap.add_argument("--no-prefill", action="store_true", help="skip the M=8192 prefill measurements")
    ap.add_argument("--no-moe", action="store_true", help="skip the MoE bank measurement")
    ap.add_argument("--no-mlp", action="store_true", help="skip the dense MLP block measurement")
    ap.add_argument("--no-embed", action="store_true", help="skip the int8 embedding gather and output-head measurements")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured streaming-read and MFMA peaks")
    ap.add_argument("--no-int8-decode", action="store_true",
                    help="skip the 8-bit activation path at decode sizes (gate_up at M = 1 and 8)")
    ap.add_argument("--sweep", action="store_true",
                    help="the M sweep over a 64-layer projection set on both paths (prints its own report)")
    ap.add_argument("--sweep-ms", default="1,4,8,16,24,32,48,64,128,512,8192")
    ap.add_argument("--pmc-prefill", action="store_true",
                    help="counter runs: 1 GiB device copies (known bytes), then two eager calls of each prefill projection")
    ap.add_argument("--pmc-ref", action="store_true",
                    help="eager decode launches (no graph) plus a plain 1 GiB copy, for hardware-counter runs")
    ap.add_argument("--pmc-moe", action="store_true",
                    help="counter runs: 1 GiB device copies (known bytes), then eager MoE bank calls at T=256 and "
                         "T=4096 (3 of each, on one bank)")
    ap.add_argument("--pmc-int8", action="store_true",
                    help="counter runs: 1 GiB device copies (known bytes), then eager int8 embedding gathers "
                         "(T=8192) and output-head calls (M=1) over the 248,320 x 5120 table")
    return ap.parse_args()


def sources_sha() -> str:
    h = hashlib.sha256()
    for p in TRAFFIC_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def stored_traffic():
    """HBM bytes per launch of the decode kernel from the committed counter summary, or None when the
    summary is missing or the kernel sources changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_sha = re.search(r"sources_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.]+)", text)
    if not m_sha or not m_b or m_sha.group(1) != sources_sha():
        return None
    return float(m_b.group(1))


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


def graph_time(torch, step, steps, warmup, reps=20, chunk=16):
    """Time calls of step(i) replayed from captured graphs, with events recorded on the current stream (the
    stream the kernels are launched on).
      * headline: `warmup` untimed calls, then exactly `steps` calls in one graph, one replay between two
        events, synchronized before and after: "mean" = seconds per call;
      * spread: a graph of `chunk` calls replayed `reps` times (at least 20), each replay between its own
        events (enqueued back to back, so the GPU does not wait on the host): "median", "p10", "p90" of the
        per-replay seconds per call."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = {}
    for n in sorted({warmup, steps, chunk}):
        if n <= 0:
            continue
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(i)
        graphs[n] = g
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    if warmup > 0:
        graphs[warmup].replay()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    graphs[steps].replay()
    t1.record(stream)
    torch.cuda.synchronize()
    mean = t0.elapsed_time(t1) / 1e3 / steps
    graphs[chunk].replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    ev[0].record(stream)
    for r in range(reps):
        graphs[chunk].replay()
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    per = np.array([ev[r].elapsed_time(ev[r + 1]) / 1e3 / chunk for r in range(reps)])
    return {"mean": mean, "median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
            "p90": float(np.percentile(per, 90)), "replays": reps, "calls_per_replay": chunk}


def stats_us(t):
    return {"median_us": round(t["median"] * 1e6, 3), "p10_us": round(t["p10"] * 1e6, 3),
            "p90_us": round(t["p90"] * 1e6, 3), "replays": t["replays"],
            "calls_per_replay": t.get("calls_per_replay", 1)}


def time_decode(torch, exl3, dev, x, out, sets, steps, warmup, flags=0):
    M, IC = x.shape
    ws = exl3.alloc_workspace(max(exl3.linear_multi_workspace_bytes(M, IC, s, flags) for s in sets), dev)
    return graph_time(torch, lambda i: exl3.linear_multi_into(out, x, sets[i % len(sets)], flags=flags, ws=ws),
                      steps, warmup)


def time_mlp(torch, exl3, synth, dev, copies=8, steps=64):
    """Dense MLP block of one decoder layer (hidden 5120, intermediate 17408; gate K=2, up K=3, down K=3) at
    decode sizes M = 1 and 8: merged gate_up, SiLU * mul, down, over `copies` weight sets in turn (89 MB of
    trellis words each, beyond the last-level cache).  Returns ({M: timing dict}, trellis bytes per
    call = 5120 * 17408 * (2 + 3 + 3) / 8)."""
    H, I = 5120, 17408
    sets = []
    for r in range(copies):
        c = synth.mlp_case(6000 + r, 1, H, I, 2, 3, 3)
        s_in = torch.from_numpy(c["gate"]["s_in"]).to(dev)
        rin = torch.from_numpy(c["gate"]["rin"]).to(dev)
        one = []
        for key in ("gate", "up", "down"):
            p = c[key]
            t = {k: torch.from_numpy(p[k]).to(dev) for k in ("code", "rout", "s_out", "s_in", "rin")}
            if key != "down":
                t.update(s_in=s_in, rin=rin)
            t["K"] = p["K"]
            one.append(t)
        sets.append(one)
    tbytes = H * I * (2 + 3 + 3) // 8
    res = {}
    for M in (1, 8):
        x = torch.randn((M, H), device=dev).to(torch.bfloat16)
        out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
        ws = exl3.alloc_workspace(exl3.mlp_workspace_bytes(M, H, I, sets[0][0], sets[0][1]), dev)
        t = graph_time(torch, lambda i: exl3.mlp_forward(x, *sets[i % copies], out=out, ws=ws), steps, copies)
        sec = t["median"]
        res[M] = t
        print(f"# mlp H={H} I={I} M={M}: {sec * 1e6:.2f} us/call (median), {tbytes / sec / 1e9:.1f} GB/s trellis",
              file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res, tbytes


def time_prefill(torch, exl3, synth, dev, reps=20):
    """M=8192 prefill projections: gate_up (IC=5120 -> 2 x 17408, K=2 | K=3) and down (17408 -> 5120, K=3),
    each on the 16-bit and on the 8-bit activation path, `reps` eager calls each between events.  Returns
    {name: (timing dict as graph_time's, FLOP per call)}; FLOP = 2*M*IC*OC (decode and transforms not
    counted)."""
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
        for tag, flags in (("", 0), ("_int8", exl3.ACT_INT8)):
            ws = exl3.alloc_workspace(exl3.linear_multi_workspace_bytes(M, IC, sh, flags), dev)
            for _ in range(2):
                exl3.linear_multi_into(out, x, sh, flags=flags, ws=ws)
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
            ev[0].record(stream)
            for r in range(reps):
                exl3.linear_multi_into(out, x, sh, flags=flags, ws=ws)
                ev[r + 1].record(stream)
            torch.cuda.synchronize()
            per = np.array([ev[r].elapsed_time(ev[r + 1]) / 1e3 for r in range(reps)])
            t = {"mean": ev[0].elapsed_time(ev[-1]) / 1e3 / reps, "median": float(np.median(per)),
                 "p10": float(np.percentile(per, 10)), "p90": float(np.percentile(per, 90)), "replays": reps}
            res[name + tag] = (t, 2.0 * M * IC * col)
            print(f"# prefill {name}{tag} M={M}: {t['median'] * 1e3:.3f} ms/call (median of {reps}), "
                  f"{res[name + tag][1] / t['median'] / 1e12:.1f} TFLOP/s", file=sys.stderr, flush=True)
            del ws
        del x, out, sh
    return res


def time_moe(torch, exl3, synth, dev, steps=60):
    """MoE bank T=256, E=128, top-8, H=2048, I=768, K in {2,3,4}: 3 banks rotated (~665 MB of trellis)."""
    from moe_exl3_pre_amd.bank import DeviceBank, pack_bank
    cfg = synth.MOE
    banks = []
    for r in range(MOE_COPIES):
        m = synth.moe_case(1003 + r, T=cfg["T"], E=cfg["E"], topk=cfg["topk"], H=cfg["H"], I=cfg["I"], Ks=cfg["Ks"])
        banks.append(DeviceBank(pack_bank(m["experts"], cfg["H"], cfg["I"]), dev))
        if r == 0:
            x = torch.from_numpy(m["x_bits"].view(np.int16).copy()).to(dev).view(torch.bfloat16)
            ids = torch.from_numpy(m["topk_ids"].astype(np.int32)).to(dev)
            w = torch.from_numpy(m["topk_w"].astype(np.float32)).to(dev)
            used = np.unique(m["topk_ids"])
    # trellis of the experts the routing touches, averaged over the rotated banks (their K draws differ)
    tb = sum(b.packed.trellis_bytes([int(b.packed.perm[e]) for e in used]) for b in banks) / MOE_COPIES
    out = torch.empty_like(x)
    ws = exl3.alloc_workspace(exl3.moe_workspace_bytes(banks[0], cfg["T"], cfg["topk"]), dev)
    tm = graph_time(torch, lambda i: exl3.moe_bank_forward(out, x, ids, w, banks[i % MOE_COPIES], ws=ws), steps,
                    MOE_COPIES * 2)
    sec = tm["median"]
    print(f"# moe T={cfg['T']} E={cfg['E']} top{cfg['topk']}: {sec * 1e6:.1f} us/call, "
          f"{tb / sec / 1e9:.1f} GB/s trellis ({tb / 1e6:.1f} MB touched)", file=sys.stderr, flush=True)
    # a prefill-sized batch on the same banks: T = 4096 tokens (32,768 routed pairs; the route's counting
    # sort); MFMA-bound, so reported as TFLOP/s of the experts' products, 2 * pairs * (2 H I + I H)
    T = 4096
    rng = np.random.default_rng(1009)
    xp = torch.from_numpy(synth.random_activations(rng, T, cfg["H"])[1].view(np.int16).copy()).to(dev)
    xp = xp.view(torch.bfloat16)
    pid, pw = synth.routing(rng, T, cfg["E"], cfg["topk"])
    pid = torch.from_numpy(pid.astype(np.int32)).to(dev)
    pw = torch.from_numpy(pw.astype(np.float32)).to(dev)
    outp = torch.empty_like(xp)
    wsp = exl3.alloc_workspace(exl3.moe_workspace_bytes(banks[0], T, cfg["topk"]), dev)
    tp = graph_time(torch, lambda i: exl3.moe_bank_forward(outp, xp, pid, pw, banks[i % MOE_COPIES], ws=wsp), 20,
                    MOE_COPIES)
    secp = tp["median"]
    flop = 2.0 * T * cfg["topk"] * (2 * cfg["H"] * cfg["I"] + cfg["I"] * cfg["H"])
    print(f"# moe T={T} E={cfg['E']} top{cfg['topk']}: {secp * 1e6:.1f} us/call, {flop / secp / 1e12:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    return tm, tb, (T, tp, flop)


def time_embed(torch, exl3, dev, reps=50):
    """The int8 table over the pages' vocabulary (248,320 rows of 5120, a 1.27 GB table that no cache holds),
    timed in captured graphs like the other measurements:
      - embedding gather-dequant for T = 256 and 8192 random token ids; bytes per call: T*H int8 in,
        T*H bf16 out;
      - the same table as the output head for M = 1 and 16 rows of x; bytes per call: the table (V*H), its
        scales (2V), x (2MH) and the logits (2MV)."""
    V, H = 248320, 5120
    g = torch.Generator(device=dev)
    g.manual_seed(31)
    table = torch.randint(-128, 128, (V, H), dtype=torch.int8, device=dev, generator=g)
    scale = torch.randint(0x3A00, 0x3D80, (V,), dtype=torch.int32, device=dev, generator=g).to(torch.int16)
    scale = scale.view(torch.bfloat16)
    res = {}
    for T in (256, 8192):
        # several id sets, so repeated calls do not read the same rows out of the caches
        ids = [torch.randint(0, V, (T,), dtype=torch.int32, device=dev, generator=g) for _ in range(8)]
        out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
        t = graph_time(torch, lambda i: exl3.embed_int8(table, scale, ids[i % len(ids)], out=out), reps, 8)
        sec = t["median"]
        nbytes = 3 * T * H
        res[f"embed_int8_V{V}_H{H}_T{T}"] = (t, nbytes)
        print(f"# embed_int8 V={V} H={H} T={T}: {sec * 1e6:.2f} us/call, {nbytes / sec / 1e9:.1f} GB/s",
              file=sys.stderr, flush=True)
    for M in (1, 16):
        x = torch.randn((M, H), device=dev, generator=g).to(torch.bfloat16)
        out = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
        t = graph_time(torch, lambda i: exl3.lm_head_int8(x, table, scale, out=out), 20, 4)
        sec = t["median"]
        nbytes = V * H + 2 * V + 2 * M * H + 2 * M * V
        res[f"lm_head_int8_V{V}_H{H}_M{M}"] = (t, nbytes)
        print(f"# lm_head_int8 V={V} H={H} M={M}: {sec * 1e6:.2f} us/call, {nbytes / sec / 1e9:.1f} GB/s",
              file=sys.stderr, flush=True)
    del table
    torch.cuda.empty_cache()
    return res


# ---- CPU oracle beside it: the fp64 oracle on the same M=1 step, one thread and all cores --------------
# The step's output columns are independent, so the all-cores leg runs the unchanged oracle on one share of
# each shard's 128-column blocks per worker process (spawned interpreters that import numpy and the oracle
# only) and the single-thread leg runs it on all blocks in this process.

_CPU_CASE = None


def _cpu_case():
    global _CPU_CASE
    if _CPU_CASE is None:
        from moe_exl3_pre_amd import synth
        cfg = synth.DECODE_GATE_UP
        _CPU_CASE = synth.merged_case(1001, 1, cfg["IC"], [(cfg["OC_gate"], cfg["K_gate"]), (cfg["OC_up"], cfg["K_up"])])
    return _CPU_CASE


def _cpu_part(job):
    """Part `i` of `n` of one oracle step: for each shard, its blocks [i*B/n, (i+1)*B/n) of 128 columns."""
    i, n = job
    from threadpoolctl import threadpool_limits
    from oracle import exl3_oracle as O
    case = _cpu_case()
    with threadpool_limits(limits=1):
        for s in case["shards"]:
            nb = s["OC"] // 128
            b0, b1 = i * nb // n, (i + 1) * nb // n
            if b1 <= b0:
                continue
            code = s["code"][:, 8 * b0:8 * b1]
            cols = slice(128 * b0, 128 * b1)
            O.linear(case["x"], code, s["K"], s["s_in"], s["rin"], s["rout"][cols], s["s_out"][cols])
    return i


def _host_info():
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:
        usable = os.cpu_count() or 1
    return {"nproc": os.cpu_count(), "usable_cpus": usable, "model_name": model}


def cpu_baseline(min_seconds=10.0):
    """The oracle on whole M=1 steps of the decode gate_up workload (both shards, 36.7 MB of trellis words
    each): single-threaded in this process, then on all usable cores (capped at 16, the host share of one
    GPU) as one share of the output blocks per worker.  Each leg repeats whole steps until `min_seconds`
    have passed; rates are trellis GB/s."""
    import multiprocessing as mp
    from moe_exl3_pre_amd import synth
    cfg = synth.DECODE_GATE_UP
    nbytes = cfg["IC"] * (cfg["OC_gate"] * cfg["K_gate"] + cfg["OC_up"] * cfg["K_up"]) // 8
    _cpu_case()
    _cpu_part((0, 1))                                     # first touch of the arrays, untimed
    steps, t0 = 0, time.perf_counter()
    while True:
        _cpu_part((0, 1))
        steps += 1
        dt1 = time.perf_counter() - t0
        if dt1 >= min_seconds or steps >= 50:
            break
    one = nbytes * steps / dt1 / 1e9
    host = _host_info()
    workers = max(1, min(16, host["usable_cpus"]))
    ctx = mp.get_context("spawn")
    with ctx.Pool(workers) as pool:
        pool.map(_cpu_part, [(i, workers) for i in range(workers)])      # untimed: imports and the case
        psteps, t0 = 0, time.perf_counter()
        while True:
            pool.map(_cpu_part, [(i, workers) for i in range(workers)])
            psteps += 1
            dtn = time.perf_counter() - t0
            if dtn >= min_seconds / 2 or psteps >= 200:
                break
    alln = nbytes * psteps / dtn / 1e9
    return dict(value=round(alln, 4), unit="GB/s", cores=workers, kind="oracle",
                single_thread={"value": round(one, 4), "cores": 1, "steps": steps, "seconds": round(dt1, 2)},
                all_cores={"value": round(alln, 4), "cores": workers, "steps": psteps, "seconds": round(dtn, 2)},
                host=host,
                sample=f"whole M=1 steps of the decode gate_up workload (IC=4096, 2 x 14336, K=2 | K=3; fp64 numpy "
                       f"oracle): {steps} steps on 1 thread in {dt1:.1f} s; {psteps} steps on {workers} worker "
                       f"processes (one share of the 128-column blocks each) in {dtn:.1f} s")


# ---- measured peaks: what this chip delivers, as secondary denominators -----------------------------------

def measured_peaks(torch, exl3, dev):
    """What this chip delivers: a streaming read of 4 GiB (variants of loads in flight and grid size) and
    back-to-back MFMAs (f16 16x16x32 and 32x32x16, i8 16x16x64 and 32x32x32; 4 and 8 waves per SIMD); each
    variant the median of 10 timed calls after 2 untimed, each figure the best variant."""
    res, detail = {}, {}
    stream = torch.cuda.current_stream()

    def timed(fn, n=10):
        for _ in range(2):
            fn()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
        ev[0].record(stream)
        for r in range(n):
            fn()
            ev[r + 1].record(stream)
        torch.cuda.synchronize()
        return float(np.median([ev[r].elapsed_time(ev[r + 1]) / 1e3 for r in range(n)]))

    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(8192, dtype=torch.int32, device=dev)
    best = 0.0
    for variant in (0, 1, 2):
        for blocks in (2048, 4096, 8192):
            sec = timed(lambda: exl3.probe_read(buf, sink, blocks, variant))
            gbs = buf.numel() / sec / 1e9
            detail[f"read_v{variant}_b{blocks}"] = round(gbs, 1)
            best = max(best, gbs)
    res["hbm_read_GBps"] = round(best, 1)
    del buf
    msink = torch.empty(2048 * 256, dtype=torch.float32, device=dev)
    for key, kinds in (("mfma_f16_TFLOPs", (0, 1)), ("mfma_i8_TOPs", (2, 3))):
        best = 0.0
        for kind in kinds:
            for blocks in (1024, 2048):
                flop = exl3.probe_mfma(msink, kind, 1024, blocks)
                sec = timed(lambda: exl3.probe_mfma(msink, kind, 1024, blocks))
                detail[f"mfma_k{kind}_b{blocks}"] = round(flop / sec / 1e12, 1)
                best = max(best, flop / sec / 1e12)
        res[key] = round(best, 1)
    torch.cuda.empty_cache()
    print(f"# measured peaks: {res}; variants {detail}", file=sys.stderr, flush=True)
    res["variants"] = detail
    return res


def run_sweep(torch, exl3, synth, dev, ms):
    """M sweep over one 64-layer decoder's projections (hidden 5120, intermediate 17408): every layer has
    its own seeded random trellis words and scales (generated on the GPU), so successive calls stream new
    weights.  Each (projection, M) is timed on the decode-phase path (FORCE_GEMV, 16-row launches) and on
    the MFMA path (FORCE_MFMA, with its automatic feature split): one call per layer, all 64 layers, events
    around the whole pass."""
    cfg = synth.SWEEP
    L = cfg["layers"]
    gen = torch.Generator(device=dev)
    report = []
    for pi, (name, IC, OC, K) in enumerate(cfg["projections"]):
        gen.manual_seed(1004 * 100 + pi)
        codes = [torch.randint(-32768, 32768, (IC // 16, OC // 16, 16 * K), dtype=torch.int16, device=dev,
                               generator=gen) for _ in range(L)]
        vec = lambda n: (torch.rand(n, device=dev, generator=gen) + 0.5).half()
        sgn = lambda n: (torch.randint(0, 2, (n,), device=dev, generator=gen) * 2 - 1).half()
        layers = [dict(code=c, s_in=sgn(IC), rin=vec(IC), rout=vec(OC), s_out=sgn(OC)) for c in codes]
        trellis = IC * OC * K // 8
        for M in ms:
            x = (torch.randn((M, IC), device=dev, generator=gen)).to(torch.bfloat16)
            out = torch.empty((M, OC), dtype=torch.bfloat16, device=dev)
            row = {"projection": name, "IC": IC, "OC": OC, "K": K, "M": M,
                   "mfma_splits": exl3.lib().exl3_gemm_splits(M, IC, OC)}
            for tag, flags in (("gemv", exl3.FORCE_GEMV), ("mfma", exl3.FORCE_MFMA)):
                ws = exl3.alloc_workspace(exl3.linear_workspace_bytes(M, IC, OC, flags), dev)
                step = lambda i: exl3.linear_into(out, x, layers[i % L]["code"], K, layers[i % L]["s_in"],
                                                  layers[i % L]["rin"], layers[i % L]["rout"], layers[i % L]["s_out"],
                                                  flags=flags, ws=ws)
                if M <= 128:      # launch-bound sizes: replay a captured graph of the 64 calls
                    sec = graph_time(torch, step, L, L)["mean"]
                else:
                    for i in range(L):
                        step(i)
                    torch.cuda.synchronize()
                    stream = torch.cuda.current_stream()
                    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                    t0.record(stream)
                    for i in range(L):
                        step(i)
                    t1.record(stream)
                    torch.cuda.synchronize()
                    sec = t0.elapsed_time(t1) / 1e3 / L
                row[f"{tag}_us"] = round(sec * 1e6, 2)
                row[f"{tag}_trellis_GBps"] = round(trellis / sec / 1e9, 1)
                row[f"{tag}_TFLOPs"] = round(2.0 * M * IC * OC / sec / 1e12, 2)
                del ws
            row["faster"] = "gemv" if row["gemv_us"] < row["mfma_us"] else "mfma"
            print(json.dumps(row), flush=True)
            report.append(row)
            del x, out
        del codes, layers
        torch.cuda.empty_cache()
    crossover = {}
    for name, *_ in cfg["projections"]:
        rows = [r for r in report if r["projection"] == name]
        first = next((r["M"] for r in rows if r["faster"] == "mfma"), None)
        last_gemv = max((r["M"] for r in rows if r["faster"] == "gemv"), default=None)
        crossover[name] = {"last_M_gemv_faster": last_gemv, "first_M_mfma_faster": first}
    thresholds = {name: exl3.lib().exl3_gemv_max_rows(OC) for name, IC, OC, K in cfg["projections"]}
    print(json.dumps({"sweep_crossover": crossover, "dispatch_threshold_rows": thresholds}), flush=True)


def pmc_reference(torch, exl3, dev, x, out, sets):
    """Eager launches for counter runs: 1 GiB device copies (known bytes), then decode steps."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    M, IC = x.shape
    ws = exl3.alloc_workspace(max(exl3.linear_multi_workspace_bytes(M, IC, s) for s in sets), dev)
    for i in range(4 * len(sets)):
        exl3.linear_multi_into(out, x, sets[i % len(sets)], ws=ws)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_reference": True, "copy_bytes": 1 << 30, "decode_launches": 4 * len(sets),
                      "sources_sha256_16": sources_sha()}), flush=True)


def pmc_int8(torch, exl3, dev):
    """Eager launches for counter runs over the int8 table: 1 GiB copies, 4 gathers of 8192 random ids (each
    its own id set), 4 output-head calls on one row of x."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    del src, dst
    V, H = 248320, 5120
    g = torch.Generator(device=dev)
    g.manual_seed(33)
    table = torch.randint(-128, 128, (V, H), dtype=torch.int8, device=dev, generator=g)
    scale = torch.randint(0x3A00, 0x3D80, (V,), dtype=torch.int32, device=dev, generator=g).to(torch.int16)
    scale = scale.view(torch.bfloat16)
    out = torch.empty((8192, H), dtype=torch.bfloat16, device=dev)
    for _ in range(4):
        ids = torch.randint(0, V, (8192,), dtype=torch.int32, device=dev, generator=g)
        exl3.embed_int8(table, scale, ids, out=out)
    x = torch.randn((1, H), device=dev, generator=g).to(torch.bfloat16)
    logits = torch.empty((1, V), dtype=torch.bfloat16, device=dev)
    for _ in range(4):
        exl3.lm_head_int8(x, table, scale, out=logits)
    torch.cuda.synchronize()
    print(json.dumps({"pmc_int8": True, "copy_bytes": 1 << 30, "embed_bytes": 3 * 8192 * H,
                      "head_bytes": V * H + 2 * V + 2 * H + 2 * V}), flush=True)


def pmc_moe(torch, exl3, synth, dev):
    """Eager launches for counter runs on the MoE bank: 1 GiB copies, then 3 calls at T=256 (the decode-sized
    plan) and 3 at T=4096 (the prefill plan) on one bank, with the bench's inputs."""
    from moe_exl3_pre_amd.bank import DeviceBank, pack_bank
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    del src, dst
    cfg = synth.MOE
    m = synth.moe_case(1003, T=cfg["T"], E=cfg["E"], topk=cfg["topk"], H=cfg["H"], I=cfg["I"], Ks=cfg["Ks"])
    bank = DeviceBank(pack_bank(m["experts"], cfg["H"], cfg["I"]), dev)
    rng = np.random.default_rng(1009)
    for T in (cfg["T"], 4096):
        if T == cfg["T"]:
            x = torch.from_numpy(m["x_bits"].view(np.int16).copy()).to(dev).view(torch.bfloat16)
            ids, w = m["topk_ids"], m["topk_w"]
        else:
            x = torch.from_numpy(synth.random_activations(rng, T, cfg["H"])[1].view(np.int16).copy()).to(dev)
            x = x.view(torch.bfloat16)
            ids, w = synth.routing(rng, T, cfg["E"], cfg["topk"])
        ids = torch.from_numpy(ids.astype(np.int32)).to(dev)
        w = torch.from_numpy(w.astype(np.float32)).to(dev)
        out = torch.empty_like(x)
        ws = exl3.alloc_workspace(exl3.moe_workspace_bytes(bank, T, cfg["topk"]), dev)
        for _ in range(3):
            exl3.moe_bank_forward(out, x, ids, w, bank, ws=ws)
        torch.cuda.synchronize()
        del ws
    print(json.dumps({"pmc_moe": True, "copy_bytes": 1 << 30}), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py: measures one GPU only (--gpus {a.gpus} requested); the library has no collectives "
              "or multi-GPU sharding", file=sys.stderr)
        sys.exit(2)
    import torch
    from moe_exl3_pre_amd import exl3, synth
    dev = torch.device("cuda", 0)
    exl3.lib()

    if a.sweep:
        run_sweep(torch, exl3, synth, dev, [int(m) for m in a.sweep_ms.split(",") if m])
        return
    if a.pmc_int8:
        pmc_int8(torch, exl3, dev)
        return
    if a.pmc_moe:
        pmc_moe(torch, exl3, synth, dev)
        return
    if a.pmc_prefill:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        del src, dst
        time_prefill(torch, exl3, synth, dev, reps=2)
        print(json.dumps({"pmc_prefill": True, "copy_bytes": 1 << 30}), flush=True)
        return
    IC, ldo, sets, trellis_bytes = build_gate_up(torch, dev, synth, COPIES)
    rng = np.random.default_rng(77)
    if a.pmc_ref:
        _, xb = synth.random_activations(rng, 1, IC)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        pmc_reference(torch, exl3, dev, x, torch.empty((1, ldo), dtype=torch.bfloat16, device=dev), sets)
        return
    results = {}
    for M in [1] + [int(m) for m in a.extra_m.split(",") if m]:
        _, xb = synth.random_activations(rng, M, IC)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        out = torch.empty((M, ldo), dtype=torch.bfloat16, device=dev)
        t = time_decode(torch, exl3, dev, x, out, sets, a.steps if M == 1 else max(a.steps // 4, 2 * COPIES),
                        a.warmup if M == 1 else COPIES)
        results[M] = t
        print(f"# decode gate_up M={M}: {t['mean'] * 1e6:.2f} us/step (median {t['median'] * 1e6:.2f}, p10 "
              f"{t['p10'] * 1e6:.2f}, p90 {t['p90'] * 1e6:.2f}), {trellis_bytes / t['mean'] / 1e9:.1f} GB/s trellis",
              file=sys.stderr, flush=True)
    # the 8-bit activation path at decode sizes: the pre-pass (row maxima, scales, codes) plus the decode kernel
    results_i8 = {}
    for M in () if a.no_int8_decode else (1, 8):
        _, xb = synth.random_activations(rng, M, IC)
        x = torch.from_numpy(xb.view(np.int16).copy()).to(dev).view(torch.bfloat16)
        out = torch.empty((M, ldo), dtype=torch.bfloat16, device=dev)
        t = time_decode(torch, exl3, dev, x, out, sets, max(a.steps // 4, 2 * COPIES), COPIES, flags=exl3.ACT_INT8)
        results_i8[M] = t
        print(f"# decode gate_up 8-bit M={M}: {t['mean'] * 1e6:.2f} us/step (median {t['median'] * 1e6:.2f})",
              file=sys.stderr, flush=True)

    peaks = None if a.no_peaks else measured_peaks(torch, exl3, dev)
    prefill = {} if a.no_prefill else time_prefill(torch, exl3, synth, dev)
    moe = None if a.no_moe else time_moe(torch, exl3, synth, dev)
    mlp = None if a.no_mlp else time_mlp(torch, exl3, synth, dev)
    embed = {} if a.no_embed else time_embed(torch, exl3, dev)

    def vs_measured(val, key):
        return round(val / peaks[key], 4) if peaks else None

    t1 = results[1]
    sec = t1["mean"]
    gbs = trellis_bytes / sec / 1e9
    traffic = stored_traffic()
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "decode gate_up: IC=4096, gate OC=14336 K=2 | up OC=14336 K=3, M=1, "
                               f"{COPIES} rotated weight copies", "M": 1, "IC": IC, "OC": [14336, 14336], "K": [2, 3],
                   "trellis_bytes_per_step": trellis_bytes},
        "timing": dict(stats_us(t1), mean_us=round(sec * 1e6, 3)),
        # one step is one launch of the decode kernel, so the per-step event time is its launch duration
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": DECODE_KERNEL,
                     "kernel_us": round(sec * 1e6, 3), "bytes_per_launch": trellis_bytes,
                     "frac_of_measured_read": vs_measured(gbs, "hbm_read_GBps")},
        "extra": {},
    }
    if peaks:
        line["measured_peaks"] = peaks
    for M, t in results.items():
        g = trellis_bytes / t["mean"] / 1e9
        line["extra"][f"decode_M{M}"] = dict(stats_us(t), us_per_step=round(t["mean"] * 1e6, 3), trellis_GBps=round(g, 1),
                                             frac_hbm=round(g / HBM_PEAK_GBS, 4),
                                             frac_of_measured_read=vs_measured(g, "hbm_read_GBps"))
    for M, t in results_i8.items():
        g = trellis_bytes / t["mean"] / 1e9
        line["extra"][f"decode_int8_M{M}"] = dict(stats_us(t), us_per_step=round(t["mean"] * 1e6, 3),
                                                  trellis_GBps=round(g, 1), frac_hbm=round(g / HBM_PEAK_GBS, 4))
    for name, (t, flop) in prefill.items():
        tf = flop / t["median"] / 1e12
        e = dict(stats_us(t), ms_per_call=round(t["median"] * 1e3, 4), TFLOPs=round(tf, 1),
                 frac_of_f16_peak=round(tf / F16_PEAK_TFLOPS, 4),
                 frac_of_measured_f16=vs_measured(tf, "mfma_f16_TFLOPs"))
        if name.endswith("_int8"):
            # the 8-bit path's integer codes run on the f16 MFMA (exact products); also against the int8 peak
            e.update(frac_of_i8_peak=round(tf / I8_PEAK_TOPS, 4), frac_of_measured_i8=vs_measured(tf, "mfma_i8_TOPs"))
        line["extra"][f"prefill_{name}_M8192"] = e
    if moe is not None:
        tm, tb, (Tp, tp, flp) = moe
        tf = flp / tp["median"] / 1e12
        line["extra"][f"moe_T{Tp}_E128_top8"] = dict(stats_us(tp), TFLOPs=round(tf, 1),
                                                     frac_of_f16_peak=round(tf / F16_PEAK_TFLOPS, 4))
        g = tb / tm["median"] / 1e9
        line["extra"]["moe_T256_E128_top8"] = dict(stats_us(tm), trellis_MB=round(tb / 1e6, 1), trellis_GBps=round(g, 1),
                                                   frac_hbm=round(g / HBM_PEAK_GBS, 4),
                                                   frac_of_measured_read=vs_measured(g, "hbm_read_GBps"))
    if mlp is not None:
        times, tb = mlp
        for M, t in times.items():
            g = tb / t["median"] / 1e9
            line["extra"][f"mlp_H5120_I17408_M{M}"] = dict(stats_us(t), trellis_GBps=round(g, 1),
                                                            frac_hbm=round(g / HBM_PEAK_GBS, 4))
    for key, (t, nbytes) in embed.items():
        g = nbytes / t["median"] / 1e9
        line["extra"][key] = dict(stats_us(t), GBps=round(g, 1), frac_hbm=round(g / HBM_PEAK_GBS, 4),
                                  frac_of_measured_read=vs_measured(g, "hbm_read_GBps"))
    if not a.no_cpu:
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
