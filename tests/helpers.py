"""Shared test helpers: move seeded synthetic cases to the GPU and compare against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

from oracle import exl3_oracle as O


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda", 0)


def to_dev_x(x_bits: np.ndarray) -> torch.Tensor:
    """bf16 tensor on the GPU from raw bf16 bits."""
    return torch.from_numpy(x_bits.view(np.int16).copy()).to(dev()).view(torch.bfloat16)


def to_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev())


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (n if n > 0 else 1.0))


def assert_close_linear(got: np.ndarray, ref16: np.ndarray, ref64: np.ndarray, tol: float = 1e-2):
    """Two bars.  (1) relative Frobenius error against the exact fp64 result <= tol (the layer's stated
    bound for the 16-bit path).  (2) element-wise against the oracle that rounds the rotated
    activations to fp16 as the GPU does: the remaining differences are the fp32 accumulation order and
    the final bf16 rounding, so |d| <= 2^-8 |ref| + 2^-10 rms(ref)."""
    e = rel_fro(got, ref64)
    assert e <= tol, f"relative Frobenius error {e:.3e} > {tol}"
    rms = float(np.sqrt(np.mean(ref16 ** 2))) if ref16.size else 0.0
    bound = 2.0 ** -8 * np.abs(ref16) + 2.0 ** -10 * rms
    bad = np.abs(got - ref16) > bound
    assert not bad.any(), (f"{int(bad.sum())} of {bad.size} elements outside the bf16 bound; worst "
                           f"{float(np.max(np.abs(got - ref16) - bound)):.3e}")
    return e


def shard_to_dev(s: dict, s_in=None, rin=None) -> dict:
    d = dict(code=to_dev(s["code"]), K=s["K"], col0=s.get("col0", 0), rout=to_dev(s["rout"]), s_out=to_dev(s["s_out"]))
    d["s_in"] = s_in if s_in is not None else to_dev(s["s_in"])
    d["rin"] = rin if rin is not None else to_dev(s["rin"])
    return d


def oracle_block_columns(x, code, K, s_in, rin, rout, s_out, blocks, act="f64"):
    """Oracle output restricted to whole 128-column blocks `blocks` (decodes only those tile columns)."""
    cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    tiles = np.concatenate([np.arange(8 * b, 8 * b + 8) for b in blocks])
    sub = np.ascontiguousarray(code[:, tiles])
    y = O.linear(x, sub, K, s_in, rin, np.asarray(rout)[cols], np.asarray(s_out)[cols], act=act)
    return cols, y
