"""Seeded synthetic inputs for the EXL3 linear layer and the MoE expert bank.

This module only draws random numbers and packs them into the layouts the layer consumes; it
holds none of the layer's arithmetic.  The tests feed the same arrays to the CPU oracle and to the
HIP path, and the benchmark uses it for its workloads.

Recipe (every workload):
  * code   -- int16 uniform over all 2^16 bit patterns, shape [IC/16, OC/16, 16K];
  * x      -- N(0, 1) rounded to bf16 (round to nearest even);
  * s_in, s_out -- fp16 random signs (+1 / -1 with probability 1/2);
  * rin, rout   -- fp16 U(0.5, 1.5);
  * MoE suh / svh -- fp16 sign * U(0.5, 1.5);
  * MoE routing -- gate logits N(0, 1) [T, E], softmax per row, the top-k experts by probability
    (ties to the lower id), ordered by descending probability, weights = the probabilities
    (not renormalised);  per-expert bitrate K_e uniform on {2, 3, 4}.
Generators are numpy PCG64 (`default_rng(seed)`).
"""
from __future__ import annotations

import numpy as np

# Workloads (shapes fixed by the layer's benchmark configurations).
SMALL = dict(M=4, IC=512, OC=512, K=3)                         # single projection
DECODE_GATE_UP = dict(IC=4096, OC_gate=14336, K_gate=2, OC_up=14336, K_up=3, Ms=(1, 2, 4, 8))
PREFILL = dict(M=8192, gate_up=dict(IC=5120, OC=17408, K_gate=2, K_up=3), down=dict(IC=17408, OC=5120, K=3))
MOE = dict(T=256, E=128, topk=8, H=2048, I=768, Ks=(2, 3, 4))
SWEEP = dict(layers=64, hidden=5120, inter=17408,
             projections=(("qkv", 5120, 7168, 3), ("o", 5120, 5120, 3), ("gate", 5120, 17408, 2),
                          ("up", 5120, 17408, 3), ("down", 17408, 5120, 3)),
             Ms=(1, 8, 64, 512, 8192))


def bf16_round(a) -> tuple[np.ndarray, np.ndarray]:
    """float32 -> bf16 with round-to-nearest-even.  Returns (values as float32, raw uint16 bits)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    bits = rounded.astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    return vals.reshape(a.shape), bits.reshape(a.shape)


def random_code(rng: np.random.Generator, IC: int, OC: int, K: int) -> np.ndarray:
    """Uniform random trellis words, int16 [IC/16, OC/16, 16K]."""
    return rng.integers(0, 1 << 16, size=(IC // 16, OC // 16, 16 * K), dtype=np.uint16).view(np.int16)


def random_signs(rng, n) -> np.ndarray:
    return np.where(rng.random(n) < 0.5, -1.0, 1.0).astype(np.float16)


def random_scales(rng, n) -> np.ndarray:
    return rng.uniform(0.5, 1.5, n).astype(np.float16)


def random_activations(rng, M, IC) -> tuple[np.ndarray, np.ndarray]:
    """x ~ N(0,1) rounded to bf16: (float32 values, uint16 bits), [M, IC]."""
    return bf16_round(rng.standard_normal((M, IC)).astype(np.float32))


def linear_case(seed: int, M: int, IC: int, OC: int, K: int) -> dict:
    """One projection: x, code and the four vectors."""
    rng = np.random.default_rng(seed)
    x, xb = random_activations(rng, M, IC)
    return dict(M=M, IC=IC, OC=OC, K=K, x=x, x_bits=xb, code=random_code(rng, IC, OC, K),
                s_in=random_signs(rng, IC), rin=random_scales(rng, IC),
                rout=random_scales(rng, OC), s_out=random_signs(rng, OC))


def shard(rng, IC: int, OC: int, K: int) -> dict:
    """Per-shard tensors of a merged projection (own code / rout / s_out)."""
    return dict(OC=OC, K=K, code=random_code(rng, IC, OC, K), rout=random_scales(rng, OC), s_out=random_signs(rng, OC))


def merged_case(seed: int, M: int, IC: int, shards: list[tuple[int, int]], shared_input_vectors: bool = True) -> dict:
    """Several shards (OC_i, K_i) reading one x and writing adjacent column slices of one output.
    With shared_input_vectors the shards share s_in / rin; otherwise each shard draws its own."""
    rng = np.random.default_rng(seed)
    x, xb = random_activations(rng, M, IC)
    s_in, rin = random_signs(rng, IC), random_scales(rng, IC)
    sh, col = [], 0
    for OC, K in shards:
        d = shard(rng, IC, OC, K)
        if shared_input_vectors:
            d.update(s_in=s_in, rin=rin)
        else:
            d.update(s_in=random_signs(rng, IC), rin=random_scales(rng, IC))
        d["col0"] = col
        col += OC
        sh.append(d)
    return dict(M=M, IC=IC, ldo=col, x=x, x_bits=xb, shards=sh)


def routing(rng, T: int, E: int, topk: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-k of softmax(N(0,1) logits): (ids int32 [T, topk], weights float32 [T, topk])."""
    g = rng.standard_normal((T, E))
    p = np.exp(g - g.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    order = np.lexsort((np.arange(E)[None, :].repeat(T, 0), -p), axis=1)[:, :topk]
    ids = order.astype(np.int32)
    w = np.take_along_axis(p, order, axis=1).astype(np.float32)
    return ids, w


def sign_scale(rng, shape) -> np.ndarray:
    s = np.where(rng.random(shape) < 0.5, -1.0, 1.0)
    return (s * rng.uniform(0.5, 1.5, shape)).astype(np.float16)


def moe_case(seed: int, T: int = 256, E: int = 128, topk: int = 8, H: int = 2048, I: int = 768,
             Ks=(2, 3, 4), k_d_independent: bool = False) -> dict:
    """One MoE layer: routing, activations and per-logical-expert tensors.

    experts[e] holds w1, w3 (int16 [H/16, I/16, 16 k_gu]), w2 (int16 [I/16, H/16, 16 k_d]) and the
    fp16 vectors w1_suh, w3_suh [H], w1_svh, w3_svh [I], w2_suh [I], w2_svh [H]."""
    rng = np.random.default_rng(seed)
    ids, w = routing(rng, T, E, topk)
    x, xb = random_activations(rng, T, H)
    kg = rng.choice(np.asarray(Ks), size=E)
    kd = rng.choice(np.asarray(Ks), size=E) if k_d_independent else kg
    experts = []
    for e in range(E):
        k_gu, k_d = int(kg[e]), int(kd[e])
        experts.append(dict(
            k_gu=k_gu, k_d=k_d,
            w1=random_code(rng, H, I, k_gu), w3=random_code(rng, H, I, k_gu), w2=random_code(rng, I, H, k_d),
            w1_suh=sign_scale(rng, H), w3_suh=sign_scale(rng, H),
            w1_svh=sign_scale(rng, I), w3_svh=sign_scale(rng, I),
            w2_suh=sign_scale(rng, I), w2_svh=sign_scale(rng, H)))
    return dict(T=T, E=E, topk=topk, H=H, I=I, x=x, x_bits=xb, topk_ids=ids, topk_w=w, experts=experts)


def mlp_case(seed: int, M: int, H: int, I: int, K_gate: int, K_up: int, K_down: int) -> dict:
    """A dense MLP block: gate and up over H -> I sharing s_in / rin, down over I -> H with its own."""
    rng = np.random.default_rng(seed)
    x, xb = random_activations(rng, M, H)
    s_in, rin = random_signs(rng, H), random_scales(rng, H)
    gate, up = shard(rng, H, I, K_gate), shard(rng, H, I, K_up)
    for d in (gate, up):
        d.update(s_in=s_in, rin=rin)
    down = shard(rng, I, H, K_down)
    down.update(s_in=random_signs(rng, I), rin=random_scales(rng, I))
    return dict(M=M, H=H, I=I, x=x, x_bits=xb, gate=gate, up=up, down=down)
