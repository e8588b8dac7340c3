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


def gpu_int8_codes(x_dev, s_in_dev, rin_dev, x64, s_in, rin):
    """The 8-bit codes and row scales the kernels use, read back through the rotate hook, after checking
    them against the oracle's quantize_rows_int8: scales within 2e-6 relative (fp32 against fp64 rotation),
    codes equal except by one where xh/sc lies within 1e-4 of a rounding boundary (a decision the kernel
    takes in fp32).  The hook and the GEMM's pre-pass compute xh with the same butterfly sequence, so these
    are the GEMM's own codes.  Returns (q int64 [M, IC], sc float64 [M])."""
    from moe_exl3_pre_amd import exl3
    q, sc = exl3.rotate_activations(x_dev, s_in_dev, rin_dev, int8=True)
    torch.cuda.synchronize()
    q = q.cpu().numpy().astype(np.int64)
    sc = sc.cpu().numpy().astype(np.float64)
    xh = O.rotate_input(x64, s_in, rin)
    q_ref, sc_ref = O.quantize_rows_int8(xh)
    assert np.allclose(sc, sc_ref, rtol=2e-6, atol=0), "row scales"
    assert np.abs(q).max(initial=0) <= 127
    diff = q != q_ref
    if diff.any():
        frac = (xh / np.where(sc_ref > 0, sc_ref, 1.0)[:, None]) % 1.0
        near_tie = np.abs(frac - 0.5) < 1e-4
        assert np.all(np.abs(q - q_ref)[diff] == 1) and np.all(near_tie[diff]), int(diff.sum())
    return q, sc


def oracle_int8_block_columns(q, sc, code, K, rout, s_out, blocks):
    """The oracle's 8-bit contraction and output transform on given codes, restricted to whole 128-column
    blocks `blocks`."""
    cols = np.concatenate([np.arange(128 * b, 128 * b + 128) for b in blocks])
    tiles = np.concatenate([np.arange(8 * b, 8 * b + 8) for b in blocks])
    sub = np.ascontiguousarray(code[:, tiles])
    return cols, O.linear_from_int8(q, sc, sub, K, np.asarray(rout)[cols], np.asarray(s_out)[cols])


def assert_bf16_activation(got_bits, want_bits, exact, loose=None):
    """A bf16 activation the kernel forms in fp32 against the oracle's fp64 one (want_bits = bf16 of the
    fp64 value `exact`): equal, except one unit in the last place where `exact` lies within fp32 error
    (2^-18 relative) of the midpoint between the two bf16 neighbours, i.e. where rounding fp32 and fp64
    values may legitimately differ; signed zeros compare equal.  Where `loose` is set the kernel's fp32
    intermediates are subnormal (fewer significant bits), and one unit is allowed anywhere."""
    got = np.asarray(got_bits).astype(np.int32)
    want = np.asarray(want_bits).astype(np.int32)
    sign_zero = ((got & 0x7FFF) == 0) & ((want & 0x7FFF) == 0)
    diff = (got != want) & ~sign_zero
    if diff.any():
        assert np.all(np.abs(got - want)[diff] == 1), "activation off by more than one unit"
        mid = (O.bf16_bits_to_f64(got[diff].astype(np.uint16)) + O.bf16_bits_to_f64(want[diff].astype(np.uint16))) / 2
        ex = np.asarray(exact)[diff]
        ok = np.abs(ex - mid) <= 2.0 ** -18 * np.abs(ex)
        if loose is not None:
            ok |= np.asarray(loose)[diff]
        assert np.all(ok), "activation differs away from a rounding tie"
    return int(diff.sum())


def silu_mul_refs(gu_bits, I):
    """(oracle bf16 bits, exact fp64 value, loose mask) of the activation of a bf16 gate_up [M, 2I]; the
    mask marks |silu(g)| < 2^-119, where the kernel's e^g (and so its product) is an fp32 subnormal."""
    g = O.bf16_bits_to_f64(gu_bits[:, :I])
    u = O.bf16_bits_to_f64(gu_bits[:, I:])
    sg = O.silu(g)
    return O.silu_mul_bf16(gu_bits[:, :I], gu_bits[:, I:]), sg * u, np.abs(sg) < 2.0 ** -119
