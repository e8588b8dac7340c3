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

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-prefill] [--no-moe] [--no-mlp]
                    [--no-embed]
    python bench.py --pmc-ref ...     # eager launches plus a 1 GiB copy, for counter runs
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
    ap.add_argument("--sweep", action="store_true",
                    help="the M sweep over a 64-layer projection set on both paths (prints its own report)")
    ap.add_argument("--sweep-ms", default="1,4,8,16,24,32,48,64,128,512,8192")
    ap.add_argument("--pmc-prefill", action="store_true",
                    help="counter runs: 1 GiB device copies (known bytes), then two eager calls of each prefill projection")
    ap.add_argument("--pmc-ref", action="store_true",
                    help="eager decode launches (no graph) plus a plain 1 GiB copy, for hardware-counter runs")
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


def graph_time(torch, step, steps, warmup):
    """Capture `warmup` and `steps` calls of step(i) in two graphs; return seconds per step measured with
    events on the current stream (the stream the kernels are launched on)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(3):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for n in (warmup, steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(i)
        graphs.append(g)
    torch.cuda.synchronize()
    graphs[0].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    graphs[1].replay()
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / 1e3 / steps


def time_decode(torch, exl3, dev, x, out, sets, steps, warmup):
    M, IC = x.shape
    ws = exl3.alloc_workspace(max(exl3.linear_multi_workspace_bytes(M, IC, s) for s in sets), dev)
    return graph_time(torch, lambda i: exl3.linear_multi_into(out, x, sets[i % len(sets)], ws=ws), steps, warmup)


def time_mlp(torch, exl3, synth, dev, copies=8, steps=64):
    """Dense MLP block of one decoder layer (hidden 5120, intermediate 17408; gate K=2, up K=3, down K=3) at
    decode sizes M = 1 and 8: merged gate_up, SiLU * mul, down, over `copies` weight sets in turn (89 MB of
    trellis words each, beyond the last-level cache).  Returns ({M: seconds per call}, trellis bytes per
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
        sec = graph_time(torch, lambda i: exl3.mlp_forward(x, *sets[i % copies], out=out, ws=ws), steps, copies)
        res[M] = sec
        print(f"# mlp H={H} I={I} M={M}: {sec * 1e6:.2f} us/call, {tbytes / sec / 1e9:.1f} GB/s trellis",
              file=sys.stderr, flush=True)
    del sets
    torch.cuda.empty_cache()
    return res, tbytes


def time_prefill(torch, exl3, synth, dev, reps=5):
    """M=8192 prefill projections: gate_up (IC=5120 -> 2 x 17408, K=2 | K=3) and down (17408 -> 5120, K=3),
    each on the 16-bit and on the 8-bit activation path.  Returns {name: (seconds per call, FLOP per call)};
    FLOP = 2*M*IC*OC (decode and transforms not counted)."""
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
            exl3.linear_multi_into(out, x, sh, flags=flags, ws=ws)
            torch.cuda.synchronize()
            stream = torch.cuda.current_stream()
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            t0.record(stream)
            for _ in range(reps):
                exl3.linear_multi_into(out, x, sh, flags=flags, ws=ws)
            t1.record(stream)
            torch.cuda.synchronize()
            sec = t0.elapsed_time(t1) / 1e3 / reps
            res[name + tag] = (sec, 2.0 * M * IC * col)
            print(f"# prefill {name}{tag} M={M}: {sec * 1e3:.3f} ms/call, {res[name + tag][1] / sec / 1e12:.1f} TFLOP/s",
                  file=sys.stderr, flush=True)
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
    sec = graph_time(torch, lambda i: exl3.moe_bank_forward(out, x, ids, w, banks[i % MOE_COPIES], ws=ws), steps,
                     MOE_COPIES * 2)
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
    secp = graph_time(torch, lambda i: exl3.moe_bank_forward(outp, xp, pid, pw, banks[i % MOE_COPIES], ws=wsp), 12,
                      MOE_COPIES)
    flop = 2.0 * T * cfg["topk"] * (2 * cfg["H"] * cfg["I"] + cfg["I"] * cfg["H"])
    print(f"# moe T={T} E={cfg['E']} top{cfg['topk']}: {secp * 1e6:.1f} us/call, {flop / secp / 1e12:.1f} TFLOP/s",
          file=sys.stderr, flush=True)
    return sec, tb, (T, secp, flop)


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
        sec = graph_time(torch, lambda i: exl3.embed_int8(table, scale, ids[i % len(ids)], out=out), reps, 8)
        nbytes = 3 * T * H
        res[f"embed_int8_V{V}_H{H}_T{T}"] = (sec, nbytes)
        print(f"# embed_int8 V={V} H={H} T={T}: {sec * 1e6:.2f} us/call, {nbytes / sec / 1e9:.1f} GB/s",
              file=sys.stderr, flush=True)
    for M in (1, 16):
        x = torch.randn((M, H), device=dev, generator=g).to(torch.bfloat16)
        out = torch.empty((M, V), dtype=torch.bfloat16, device=dev)
        sec = graph_time(torch, lambda i: exl3.lm_head_int8(x, table, scale, out=out), max(reps // 5, 8), 4)
        nbytes = V * H + 2 * V + 2 * M * H + 2 * M * V
        res[f"lm_head_int8_V{V}_H{H}_M{M}"] = (sec, nbytes)
        print(f"# lm_head_int8 V={V} H={H} M={M}: {sec * 1e6:.2f} us/call, {nbytes / sec / 1e9:.1f} GB/s",
              file=sys.stderr, flush=True)
    del table
    torch.cuda.empty_cache()
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
                    sec = graph_time(torch, step, L, L)
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
    if a.pmc_prefill:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        del src, dst
        time_prefill(torch, exl3, synth, dev, reps=1)
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
        sec = time_decode(torch, exl3, dev, x, out, sets, a.steps if M == 1 else max(a.steps // 4, COPIES),
                          a.warmup if M == 1 else COPIES)
        results[M] = sec
        print(f"# decode gate_up M={M}: {sec * 1e6:.2f} us/step, {trellis_bytes / sec / 1e9:.1f} GB/s trellis",
              file=sys.stderr, flush=True)

    prefill = {} if a.no_prefill else time_prefill(torch, exl3, synth, dev)
    moe = None if a.no_moe else time_moe(torch, exl3, synth, dev)
    mlp = None if a.no_mlp else time_mlp(torch, exl3, synth, dev)
    embed = {} if a.no_embed else time_embed(torch, exl3, dev)

    sec = results[1]
    gbs = trellis_bytes / sec / 1e9
    traffic = stored_traffic()
    line = {
        "metric": METRIC, "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(sec * 1e3, 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f16", "data": "synthetic",
        "config": {"workload": "decode gate_up: IC=4096, gate OC=14336 K=2 | up OC=14336 K=3, M=1, "
                               f"{COPIES} rotated weight copies", "M": 1, "IC": IC, "OC": [14336, 14336], "K": [2, 3],
                   "trellis_bytes_per_step": trellis_bytes},
        # one step is one launch of the decode kernel, so the per-step event time is its launch duration
        "roofline": {"bound": "hbm", "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic, "kernel": DECODE_KERNEL,
                     "kernel_us": round(sec * 1e6, 3), "bytes_per_launch": trellis_bytes},
        "extra": {f"decode_M{M}": {"us_per_step": round(s * 1e6, 3), "trellis_GBps": round(trellis_bytes / s / 1e9, 1),
                                   "frac_hbm": round(trellis_bytes / s / 1e9 / HBM_PEAK_GBS, 4)}
                  for M, s in results.items()},
    }
    for name, (s, flop) in prefill.items():
        line["extra"][f"prefill_{name}_M8192"] = {"ms_per_call": round(s * 1e3, 4), "TFLOPs": round(flop / s / 1e12, 1),
                                                  "frac_of_f16_peak": round(flop / s / 1e12 / F16_PEAK_TFLOPS, 4)}
    if moe is not None:
        s, tb, (Tp, sp, flp) = moe
        line["extra"][f"moe_T{Tp}_E128_top8"] = {"us_per_call": round(sp * 1e6, 1),
                                                 "TFLOPs": round(flp / sp / 1e12, 1),
                                                 "frac_of_f16_peak": round(flp / sp / 1e12 / F16_PEAK_TFLOPS, 4)}
        line["extra"]["moe_T256_E128_top8"] = {"us_per_call": round(s * 1e6, 2), "trellis_MB": round(tb / 1e6, 1),
                                               "trellis_GBps": round(tb / s / 1e9, 1),
                                               "frac_hbm": round(tb / s / 1e9 / HBM_PEAK_GBS, 4)}
    if mlp is not None:
        times, tb = mlp
        for M, s in times.items():
            line["extra"][f"mlp_H5120_I17408_M{M}"] = {"us_per_call": round(s * 1e6, 2),
                                                        "trellis_GBps": round(tb / s / 1e9, 1),
                                                        "frac_hbm": round(tb / s / 1e9 / HBM_PEAK_GBS, 4)}
    for key, (s, nbytes) in embed.items():
        line["extra"][key] = {"us_per_call": round(s * 1e6, 2),
                                                           "GBps": round(nbytes / s / 1e9, 1),
                                                           "frac_hbm": round(nbytes / s / 1e9 / HBM_PEAK_GBS, 4)}
    if not a.no_cpu:
        from oracle import exl3_oracle as O
        line["cpu_baseline"] = cpu_baseline(synth, O)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
