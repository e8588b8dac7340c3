"""GPU parity of the dense MLP block (merged gate/up, SiLU * mul, down) against the oracle, through the C ABI.

The block's bf16 intermediates are rounding decisions that the GPU takes on fp32 values and the oracle on
fp64 values, so an intermediate may land one unit apart and then move the block's outputs by more than one
projection's bar.  The block is therefore checked step by step, each step against the oracle applied to the
GPU's own output of the step before, every element at the single projection's bar:
  1. gate_up = the merged call (also compared with the block's output chain: the block equals the three
     calls bit for bit), against the oracle's two projections of x;
  2. h = bf16(silu(g) * u) from the activation kernel, against the oracle's silu_mul_bf16 of the GPU's
     gate_up (one unit apart only next to a rounding tie);
  3. the block's output, against the oracle's down projection of the GPU's h.
On the 8-bit path each projection is compared on the kernel's own codes (see test_int8_gpu.py).  Where the
whole block fits the oracle, the relative Frobenius error against the all-oracle block is also bounded by
1e-2 (3e-2 on the 8-bit path)."""
import numpy as np
import pytest
import torch

from oracle import exl3_oracle as O
from moe_exl3_pre_amd import exl3, synth
from tests.helpers import (assert_bf16_activation, assert_close_linear, bf16_to_f64, dev, gpu_int8_codes, log,
                           oracle_block_columns, oracle_int8_block_columns, rel_fro, shard_to_dev, silu_mul_refs,
                           to_dev, to_dev_x)

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _oracle_args(p):
    return dict(code=p["code"], K=p["K"], s_in=p["s_in"], rin=p["rin"], rout=p["rout"], s_out=p["s_out"])


def _to_dev_case(c):
    s_in, rin = to_dev(c["gate"]["s_in"]), to_dev(c["gate"]["rin"])
    return (to_dev_x(c["x_bits"]), shard_to_dev(c["gate"], s_in, rin), shard_to_dev(c["up"], s_in, rin),
            shard_to_dev(c["down"]))


def _blocks(nblk, rng, n):
    """All 128-column blocks when n is None, else the first, the last and n random ones."""
    if n is None or nblk <= n + 2:
        return list(range(nblk))
    return sorted(set([0, nblk - 1] + list(rng.choice(nblk, n, replace=False))))


def _check_projection(x64, x_dev, p, p_dev, got, int8, blocks):
    """One projection's output columns `blocks` against the oracle (16-bit: fp16 operands; 8-bit: on the
    kernel's own codes of x) at the element bar; the exact fp64 projection bounds the Frobenius error."""
    cols, y64 = oracle_block_columns(x64, p["code"], p["K"], p["s_in"], p["rin"], p["rout"], p["s_out"], blocks)
    if int8:
        q, sc = gpu_int8_codes(x_dev, p_dev["s_in"], p_dev["rin"], x64, p["s_in"], p["rin"])
        _, yq = oracle_int8_block_columns(q, sc, p["code"], p["K"], p["rout"], p["s_out"], blocks)
        return assert_close_linear(got[:, cols], yq, y64, tol=3e-2)
    _, y16 = oracle_block_columns(x64, p["code"], p["K"], p["s_in"], p["rin"], p["rout"], p["s_out"], blocks,
                                  act="f16")
    return assert_close_linear(got[:, cols], y16, y64)


def _check_block(c, M, flags=0, n_blocks=None, seed=0):
    """Run the block and its three calls; check the chain step by step.  Returns (out, h) on the GPU."""
    x, g, u, d = _to_dev_case(c)
    I = c["I"]
    int8 = bool(flags & exl3.ACT_INT8)
    out = exl3.mlp_forward(x, g, u, d, flags=flags)
    gu = torch.empty((M, 2 * I), dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(gu, x, [dict(g, col0=0), dict(u, col0=I)], flags=flags)
    h = exl3.silu_mul(gu)
    ref = torch.empty_like(out)
    exl3.linear_into(ref, h, d["code"], d["K"], d["s_in"], d["rin"], d["rout"], d["s_out"], flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "the block differs from its three calls"
    rng = np.random.default_rng(seed)
    gu64 = bf16_to_f64(gu)
    # 1. gate and up
    for name, p, p_dev, col0 in (("gate", c["gate"], g, 0), ("up", c["up"], u, I)):
        e = _check_projection(c["x"], x, p, p_dev, gu64[:, col0:col0 + I], int8, _blocks(I // 128, rng, n_blocks))
        log(f"  {name}: rel err vs exact {e:.3e}")
    # 2. the activation on the GPU's own gate_up
    want, exact, loose = silu_mul_refs(_bits(gu), I)
    flips = assert_bf16_activation(_bits(h), want, exact, loose)
    # 3. down on the GPU's own h
    h64 = bf16_to_f64(h)
    e = _check_projection(h64, h, c["down"], d, bf16_to_f64(out), int8, _blocks(c["H"] // 128, rng, n_blocks))
    log(f"  down: rel err vs exact {e:.3e}; {flips} activation values one unit apart at ties")
    return out, h


def test_silu_mul_against_oracle():
    """fp32 silu on bf16 inputs, one bf16 rounding: equal to the fp64 oracle except where the exact value
    lies within fp32 error of a bf16 rounding boundary (then one unit in the last place)."""
    rng = np.random.default_rng(80)
    M, I = 7, 1024
    gu = rng.normal(scale=3.0, size=(M, 2 * I))
    gu[0, :8] = [0.0, -0.0, 60.0, -60.0, 1e-3, -1e-3, 8.0, -8.0]
    gu[1, :8] = [-88.0, -89.0, -90.0, -95.0, -100.0, -104.0, -120.0, -300.0]   # e^-|g| near and past fp32 range
    gu[1, I:I + 8] = [3.0, -3.0, 70.0, -70.0, 200.0, 700.0, 1e4, 1e30]
    gu_bits = O.f64_to_bf16_bits(gu)
    got = _bits(exl3.silu_mul(to_dev_x(gu_bits)))
    torch.cuda.synchronize()
    flips = assert_bf16_activation(got, *silu_mul_refs(gu_bits, I))
    log(f"  {flips} of {got.size} values one unit apart at rounding ties")


@pytest.mark.parametrize("M", [1, 4, 8, 40, 200])
def test_mlp_against_oracle(M):
    """H = 512, I = 1024, gate K=2, up K=3, down K=3: the decode-phase kernel up to 128 rows, the GEMM above."""
    c = synth.mlp_case(81 + M, M, 512, 1024, 2, 3, 3)
    log(f"mlp H=512 I=1024 M={M}")
    out, _ = _check_block(c, M)
    args = [_oracle_args(c[k]) for k in ("gate", "up", "down")]
    e = rel_fro(bf16_to_f64(out), O.mlp_forward(c["x"], *args))
    log(f"  block rel err vs the all-oracle block {e:.3e}")
    assert e <= 1e-2


@pytest.mark.parametrize("M", [3, 200])
def test_mlp_equals_the_three_calls(M):
    """The block is bitwise the merged gate_up call, the activation hook and the down call made one by one."""
    c = synth.mlp_case(90 + M, M, 512, 1024, 3, 2, 4)
    x, g, u, d = _to_dev_case(c)
    out = exl3.mlp_forward(x, g, u, d)
    gu = torch.empty((M, 2048), dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(gu, x, [dict(g, col0=0), dict(u, col0=1024)])
    h = exl3.silu_mul(gu)
    ref = torch.empty_like(out)
    exl3.linear_into(ref, h, d["code"], d["K"], d["s_in"], d["rin"], d["rout"], d["s_out"])
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


def test_mlp_batch_invariant_flag():
    """EXL3_BATCH_INVARIANT through the block: a row of an M=70 call equals that row run alone, for a
    block whose default dispatch switches gate_up to the GEMM above 32 rows (I = 5120)."""
    M = 70
    c = synth.mlp_case(97, M, 256, 5120, 2, 3, 3)
    x, g, u, d = _to_dev_case(c)
    assert exl3.lib().exl3_gemv_max_rows(5120) == 32
    f = exl3.BATCH_INVARIANT
    full = exl3.mlp_forward(x, g, u, d, flags=f)
    for r in (0, 1, 31, 32, 33, 69):
        one = exl3.mlp_forward(x[r:r + 1].contiguous(), g, u, d, flags=f)
        torch.cuda.synchronize()
        assert torch.equal(one[0], full[r]), r
    for m in (4, 5, 40):
        part = exl3.mlp_forward(x[:m].contiguous(), g, u, d, flags=f)
        torch.cuda.synchronize()
        assert torch.equal(part, full[:m]), m


def test_mlp_rejects_mismatched_shapes():
    c = synth.mlp_case(95, 2, 512, 1024, 2, 3, 3)
    x, g, u, d = _to_dev_case(c)
    with pytest.raises(ValueError):                       # the binding checks down's shape (I -> H)
        exl3.mlp_forward(x, g, u, g)


@pytest.mark.parametrize("M", [1, 8])
def test_mlp_decoder_shapes_against_oracle(M):
    """One decoder layer's block at full size (hidden 5120, intermediate 17408; gate K=2, up K=3, down K=3):
    every step against the oracle on sampled 128-column blocks (the first, the last and three more of each
    projection; the activation over every element)."""
    c = synth.mlp_case(96 + M, M, 5120, 17408, 2, 3, 3)
    log(f"mlp H=5120 I=17408 M={M}")
    out, _ = _check_block(c, M, n_blocks=3, seed=M)
    assert out.float().abs().max() > 0


@pytest.mark.parametrize("M", [2, 40])
def test_mlp_int8_path(M):
    """EXL3_ACT_INT8: every projection takes per-row 8-bit activations (on the GEMM) and the activation is
    written out for down's 8-bit pre-pass.  Bitwise equal to the three 8-bit calls; each step against the
    oracle on the kernel's own codes; the block within 3e-2 of the all-oracle 8-bit block."""
    c = synth.mlp_case(120 + M, M, 512, 1024, 2, 3, 3)
    log(f"mlp int8 M={M}")
    out, _ = _check_block(c, M, flags=exl3.ACT_INT8)
    args = [_oracle_args(c[k]) for k in ("gate", "up", "down")]
    e = rel_fro(bf16_to_f64(out), O.mlp_forward(c["x"], *args))
    log(f"  block rel err vs the all-oracle block {e:.3e}")
    assert e < 3e-2
