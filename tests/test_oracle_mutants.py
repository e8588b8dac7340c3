"""The oracle's pins catch plausible mistakes.

Each case below plants one mistake in a copy of the oracle's source (a wrong constant, index, operand order,
rounding rule or rounding point) and runs the pins of test_oracle.py against that copy, in this process.
At least one pin must fail for every case; the unchanged source must pass all of them the same way.
Nothing here touches the GPU or the HIP library.
"""
import inspect
import os
import types

import pytest

from tests import test_oracle as PINS

SOURCE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "exl3_oracle.py")

# name -> (text in the oracle's source, replacement)
MUTANTS = {
    "codebook multiplier": ("bits = (((s * 0x9E37) & 0xFFFF)", "bits = (((s * 0x9E35) & 0xFFFF)"),
    "codebook mask": ("& 0x8F80) | 0x3000", "& 0x8F00) | 0x3000"),
    "codebook bias": ("& 0x8F80) | 0x3000", "& 0x8F80) | 0x3800"),
    "no tail-biting wrap": ("w1 = (w0 + 1) % nwords", "w1 = np.minimum(w0 + 1, nwords - 1)"),
    "word halves swapped": ("u32 = u16[:, 0::2] | (u16[:, 1::2] << np.uint64(16))",
                            "u32 = u16[:, 1::2] | (u16[:, 0::2] << np.uint64(16))"),
    "state offset off by one": ("offs = np.arange(STATES, dtype=np.int64) * K",
                                "offs = np.arange(STATES, dtype=np.int64) * K + 1"),
    "15-bit states": ("states = (pair >> sh) & np.uint64(0xFFFF)", "states = (pair >> sh) & np.uint64(0x7FFF)"),
    "tile transposed": ("W[a0:a1] = v.transpose(0, 3, 1, 2)", "W[a0:a1] = v.transpose(0, 2, 1, 3)"),
    "Hadamard not normalised": ("return H / np.sqrt(HAD)", "return H"),
    "other Hadamard sign layout": ("H = np.block([[H, H], [H, -H]])", "H = np.block([[H, H], [-H, H]])"),
    "output scales before the Hadamard": (
        "    Z = had128(Y, axis=-1)\n    return Z * np.asarray(rout, dtype=np.float64) * np.asarray(s_out, dtype=np.float64)",
        "    Z = had128(Y * np.asarray(rout, dtype=np.float64) * np.asarray(s_out, dtype=np.float64), axis=-1)\n"
        "    return Z"),
    "input scales after the Hadamard": (
        "    t = x * np.asarray(s_in, dtype=np.float64) * np.asarray(rin, dtype=np.float64)\n    return had128(t, axis=-1)",
        "    return had128(x, axis=-1) * np.asarray(s_in, dtype=np.float64) * np.asarray(rin, dtype=np.float64)"),
    "fp16 rounding before the Hadamard": (
        "        Y = round_fp16(xh) @ W",
        "        Y = had128(round_fp16(np.asarray(x, dtype=np.float64) * np.asarray(s_in, dtype=np.float64)"
        " * np.asarray(rin, dtype=np.float64)), axis=-1) @ W"),
    "int8 scale amax/128": ("    sc = amax / 127.0", "    sc = amax / 128.0"),
    "int8 ties rounded up": ("q = np.clip(np.rint(xh / safe[..., None]), -127, 127)",
                             "q = np.clip(np.floor(xh / safe[..., None] + 0.5), -127, 127)"),
    "int8 row scale dropped": ("return output_transform(sc[:, None] * (q @ W), rout, s_out)",
                               "return output_transform((q @ W), rout, s_out)"),
    "MoE weight of the first slot": ("np.add.at(out, tok, w[tok, slot][:, None] * y)",
                                     "np.add.at(out, tok, w[tok, 0][:, None] * y)"),
    "gate and up swapped": ("    a = silu(h1) * h3", "    a = silu(h3) * h1"),
    "SiLU sign": ("return h / (1.0 + np.exp(-h))", "return h / (1.0 + np.exp(h))"),
    "bf16 by truncation": ("r = np.ldexp(np.rint(np.ldexp(v, -unit)), unit)",
                           "r = np.ldexp(np.trunc(np.ldexp(v, -unit)), unit)"),
    "embedding ids clamped": ("    ok = (ids >= 0) & (ids < V)\n    rows[ok]",
                              "    ids = np.clip(ids, 0, V - 1)\n    ok = (ids >= 0) & (ids < V)\n    rows[ok]"),
    "MLP gate and up not rounded": (
        "        h = bf16_bits_to_f64(silu_mul_bf16(f64_to_bf16_bits(g), f64_to_bf16_bits(u)))",
        "        h = bf16_bits_to_f64(f64_to_bf16_bits(silu(g) * u))"),
}


def _load(source: str) -> types.ModuleType:
    mod = types.ModuleType("exl3_oracle_under_test")
    mod.__file__ = SOURCE
    exec(compile(source, SOURCE, "exec"), mod.__dict__)
    return mod


def _pin_calls():
    """Every pin of test_oracle.py as (name, zero-argument callable), parametrised ones expanded."""
    calls = []
    for name, fn in inspect.getmembers(PINS, inspect.isfunction):
        if not name.startswith("test_") or fn.__module__ != PINS.__name__:
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((name, fn))
            continue
        (mark,) = marks
        argnames = [a.strip() for a in mark.args[0].split(",")] if isinstance(mark.args[0], str) else list(mark.args[0])
        for values in mark.args[1]:
            values = values if len(argnames) > 1 else (values,)
            calls.append((f"{name}{list(values)}", lambda fn=fn, kw=dict(zip(argnames, values)): fn(**kw)))
    return calls


def _failing_pins(module, monkeypatch, stop_at_first: bool):
    monkeypatch.setattr(PINS, "O", module)
    failed = []
    for name, call in _pin_calls():
        try:
            call()
        except Exception:   # an assertion, or the mistake breaking the computation outright
            failed.append(name)
            if stop_at_first:
                break
    return failed


def test_unchanged_oracle_passes_every_pin_in_this_harness(monkeypatch):
    with open(SOURCE) as f:
        failed = _failing_pins(_load(f.read()), monkeypatch, stop_at_first=False)
    assert not failed, failed


@pytest.mark.parametrize("name", list(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    old, new = MUTANTS[name]
    with open(SOURCE) as f:
        source = f.read()
    assert source.count(old) == 1, f"the text to change is not unique in the oracle ({name})"
    failed = _failing_pins(_load(source.replace(old, new)), monkeypatch, stop_at_first=True)
    assert failed, f"no pin fails with the mistake '{name}' planted"
