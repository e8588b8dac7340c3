"""GPU parity of the 8-bit activation path (EXL3_ACT_INT8) through the C ABI.

The codes are a decision the kernel takes in fp32 and the oracle in fp64, so they may differ by one where
xh/sc lies next to a rounding boundary.  Each test therefore (1) checks the kernel's codes and row scales
against the oracle's quantize_rows_int8 (equal except such near-ties), then (2) runs the oracle's
contraction and output transform on the kernel's own codes and compares every output element at the
16-bit path's bar, and (3) bounds the relative Frobenius error against the exact fp64 layer by 3e-2."""
import numpy as np
import pytest
import torch

from oracle import exl3_oracle as O
from moe_exl3_pre_amd import exl3, synth
from tests.helpers import (assert_close_linear, bf16_to_f64, dev, gpu_int8_codes, log, oracle_block_columns,
                           oracle_int8_block_columns, shard_to_dev, to_dev, to_dev_x)

pytestmark = pytest.mark.gpu

TOL_INT8 = 3e-2
SENTINEL = -1000.0


def _dev_case(c):
    return dict(x=to_dev_x(c["x_bits"]), code=to_dev(c["code"]), s_in=to_dev(c["s_in"]), rin=to_dev(c["rin"]),
                rout=to_dev(c["rout"]), s_out=to_dev(c["s_out"]))


def _run(c, d, flags=exl3.ACT_INT8, ldo=None, col0=0, x=None):
    x = d["x"] if x is None else x
    out = torch.full((x.shape[0], ldo or c["OC"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_into(out, x, d["code"], c["K"], d["s_in"], d["rin"], d["rout"], d["s_out"], col0=col0, flags=flags)
    torch.cuda.synchronize()
    return out


def _refs(c, d, rows=None):
    """(oracle on the kernel's own codes, exact fp64 layer) for the rows `rows` (all by default)."""
    rows = np.arange(c["M"]) if rows is None else np.asarray(rows)
    x = c["x"][rows]
    xd = d["x"][torch.from_numpy(rows).to(dev())].contiguous()
    q, sc = gpu_int8_codes(xd, d["s_in"], d["rin"], x, c["s_in"], c["rin"])
    args = (c["code"], c["K"], c["s_in"], c["rin"], c["rout"], c["s_out"])
    return O.linear_from_int8(q, sc, c["code"], c["K"], c["rout"], c["s_out"]), O.linear(x, *args)


@pytest.mark.parametrize("M,IC", [(1, 512), (7, 1024), (64, 256), (333, 640)])
def test_codes_and_scales_match_the_oracle(M, IC):
    """q and the row scale from the rotate hook against quantize_rows_int8 of the oracle's rotation
    (equal except by one at near-ties; the check is in gpu_int8_codes)."""
    c = synth.linear_case(8100 + M, M, IC, 128, 2)
    d = _dev_case(c)
    q, sc = gpu_int8_codes(d["x"], d["s_in"], d["rin"], c["x"], c["s_in"], c["rin"])
    assert q.shape == (M, IC) and sc.shape == (M,)
    q_ref, _ = O.quantize_rows_int8(O.rotate_input(c["x"], c["s_in"], c["rin"]))
    log(f"  {int((q != q_ref).sum())} of {q.size} codes differ by one at near-ties")


@pytest.mark.parametrize("M", [1, 4, 17, 200, 300])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_int8_linear_ragged(M, K):
    c = synth.linear_case(8200 + 7 * M + K, M, 384, 384, K)
    d = _dev_case(c)
    out = _run(c, d)
    ref8, ref = _refs(c, d)
    e = assert_close_linear(bf16_to_f64(out), ref8, ref, tol=TOL_INT8)
    log(f"  M={M} K={K}: rel err vs exact {e:.3e}")


def test_int8_other_k_and_slice():
    for K in (1, 5, 8):
        c = synth.linear_case(8300 + K, 40, 256, 256, K)
        d = _dev_case(c)
        out = _run(c, d, ldo=640, col0=128)
        o = bf16_to_f64(out)
        assert np.all(o[:, :128] == SENTINEL) and np.all(o[:, 384:] == SENTINEL)
        ref8, ref = _refs(c, d)
        assert_close_linear(o[:, 128:384], ref8, ref, tol=TOL_INT8)


def test_int8_zero_rows_and_scale_invariance():
    c = synth.linear_case(8400, 48, 512, 256, 3)
    c["x"][5] = 0.0
    c["x_bits"][5] = 0
    d = _dev_case(c)
    base = _run(c, d)
    assert torch.all(base[5] == 0)
    # x -> 2x: the codes are unchanged and the scale doubles exactly, so the output doubles bit for bit
    twice = _run(c, d, x=(d["x"].float() * 2).to(torch.bfloat16))
    assert torch.equal(twice, (base.float() * 2).to(torch.bfloat16))


def test_int8_dispatch_and_merged():
    """The 8-bit path is dispatched by M like the 16-bit one: up to exl3_gemv_max_rows(OC) it runs the
    decode-phase kernel (bitwise equal to forcing it), above it the MFMA GEMM; merged shards equal separate
    calls bit for bit."""
    c = synth.linear_case(8500, 5, 512, 256, 2)
    d = _dev_case(c)
    assert 5 <= exl3.lib().exl3_gemv_max_rows(256)
    assert torch.equal(_run(c, d), _run(c, d, flags=exl3.ACT_INT8 | exl3.FORCE_GEMV))
    big = synth.linear_case(8502, 300, 512, 256, 2)
    assert 300 > exl3.lib().exl3_gemv_max_rows(256)
    db = _dev_case(big)
    assert torch.equal(_run(big, db), _run(big, db, flags=exl3.ACT_INT8 | exl3.FORCE_MFMA))
    case = synth.merged_case(8501, 9, 512, [(256, 2), (384, 3)])
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    shards = [shard_to_dev(s, s_in, rin) for s in case["shards"]]
    merged = torch.zeros((9, case["ldo"]), dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(merged, x, shards, flags=exl3.ACT_INT8)
    sep = torch.zeros_like(merged)
    for s in shards:
        exl3.linear_into(sep, x, s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], col0=s["col0"],
                         flags=exl3.ACT_INT8)
    torch.cuda.synchronize()
    assert torch.equal(merged, sep)


@pytest.mark.parametrize("M", [1, 3, 16, 17, 32, 40])
@pytest.mark.parametrize("K", [2, 3])
def test_int8_decode_phase_against_the_oracle(M, K):
    """The decode-phase kernel on the 8-bit path (EXL3_FORCE_GEMV): one 16-row group, two groups in one
    launch (17..32 rows) and two launches (40 rows), element by element on the kernel's own codes; the
    forced GEMM gives the same values to rounding."""
    c = synth.linear_case(8600 + 10 * M + K, M, 1024, 384, K)
    d = _dev_case(c)
    out = _run(c, d, flags=exl3.ACT_INT8 | exl3.FORCE_GEMV)
    ref8, ref = _refs(c, d)
    e = assert_close_linear(bf16_to_f64(out), ref8, ref, tol=TOL_INT8)
    gemm = bf16_to_f64(_run(c, d, flags=exl3.ACT_INT8 | exl3.FORCE_MFMA))
    assert_close_linear(bf16_to_f64(out), gemm, ref, tol=TOL_INT8)
    log(f"  M={M} K={K}: rel err vs exact {e:.3e}")


@pytest.mark.parametrize("K", [2, 3, 5])
def test_int8_inblock_codes_equal_the_codes_launch(K):
    """Launches of 1..4 rows form the codes in the decode kernel's in-block pre-pass (from the row maxima the
    first launch writes); launches of 5..32 rows read them from the codes launch.  Both quantise the same fp32
    rotated values with the same division, so a row's output is the same bits whichever path ran (a shard
    whose input-feature split is 1 at every M: IC = 1024, at most one Hadamard block per wave)."""
    c = synth.linear_case(8750 + K, 17, 1024, 2048, K)
    d = _dev_case(c)
    flags = exl3.ACT_INT8 | exl3.FORCE_GEMV
    full = _run(c, d, flags=flags)
    for M in (1, 2, 4, 5):
        part = _run(c, d, flags=flags, x=d["x"][:M].contiguous())
        assert torch.equal(part, full[:M]), M
    ref8, ref = _refs(c, d)
    assert_close_linear(bf16_to_f64(full), ref8, ref, tol=TOL_INT8)


def test_int8_decode_phase_other_k_split_and_slice():
    """K outside {2, 3, 4} (one launch per shard), a shard wide enough in IC to split along the input
    features (partials summed before the row scale), and a slice of a wider output."""
    for K, IC, OC in ((1, 512, 256), (6, 512, 256), (3, 8192, 256)):
        c = synth.linear_case(8700 + K + IC, 4, IC, OC, K)
        d = _dev_case(c)
        out = _run(c, d, flags=exl3.ACT_INT8 | exl3.FORCE_GEMV, ldo=OC + 256, col0=128)
        o = bf16_to_f64(out)
        assert np.all(o[:, :128] == SENTINEL) and np.all(o[:, 128 + OC:] == SENTINEL)
        ref8, ref = _refs(c, d)
        assert_close_linear(o[:, 128:128 + OC], ref8, ref, tol=TOL_INT8)


@pytest.mark.parametrize("M", [1, 8])
def test_int8_decode_gate_up_config_sampled(M):
    """The decode-phase gate_up shape (IC=4096, 2 x 14336, K=2 | K=3) on the 8-bit path: one merged launch
    per chunk, equal to per-shard calls bit for bit; sampled 128-column blocks of both shards against the
    oracle on the kernel's own codes."""
    cfg = synth.DECODE_GATE_UP
    case = synth.merged_case(8800 + M, M, cfg["IC"], [(cfg["OC_gate"], cfg["K_gate"]), (cfg["OC_up"], cfg["K_up"])])
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    shards = [shard_to_dev(s, s_in, rin) for s in case["shards"]]
    out = torch.full((M, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(out, x, shards, flags=exl3.ACT_INT8)
    sep = torch.full_like(out, SENTINEL)
    for s in shards:
        exl3.linear_into(sep, x, s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], col0=s["col0"],
                         flags=exl3.ACT_INT8)
    torch.cuda.synchronize()
    assert torch.equal(out, sep)
    _sampled(case["x"], x, case["shards"], shards, out, np.arange(M), 11 + M)


def _sampled(case_x, x_dev, shards, dev_shards, out, rows, seed):
    got = bf16_to_f64(out)[rows]
    rng = np.random.default_rng(seed)
    x = case_x[rows]
    xd = x_dev[torch.from_numpy(np.asarray(rows)).to(dev())].contiguous()
    codes = {}
    for s, sd in zip(shards, dev_shards):
        key = (sd["s_in"].data_ptr(), sd["rin"].data_ptr())
        if key not in codes:
            codes[key] = gpu_int8_codes(xd, sd["s_in"], sd["rin"], x, s["s_in"], s["rin"])
        q, sc = codes[key]
        nblk = s["OC"] // 128
        blocks = sorted(set([0, nblk - 1] + list(rng.choice(nblk, 2, replace=False))))
        cols, y64 = oracle_block_columns(x, s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], blocks)
        _, y8 = oracle_int8_block_columns(q, sc, s["code"], s["K"], s["rout"], s["s_out"], blocks)
        e = assert_close_linear(got[:, s["col0"] + cols], y8, y64, tol=TOL_INT8)
        log(f"  shard K={s['K']}: rel err vs exact {e:.3e}")


def test_int8_prefill_gate_up_full_size_sampled():
    p = synth.PREFILL
    cfg = p["gate_up"]
    M = p["M"]
    case = synth.merged_case(2100, M, cfg["IC"], [(cfg["OC"], cfg["K_gate"]), (cfg["OC"], cfg["K_up"])])
    log("int8 prefill gate_up 8192 x 5120 -> 2 x 17408")
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    shards = [shard_to_dev(s, s_in, rin) for s in case["shards"]]
    out = torch.full((M, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(out, x, shards, flags=exl3.ACT_INT8)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(3).choice(M, 8, replace=False)]))
    _sampled(case["x"], x, case["shards"], shards, out, rows, 4)


def test_int8_prefill_down_full_size_sampled():
    p = synth.PREFILL
    cfg = p["down"]
    M = p["M"]
    c = synth.linear_case(2101, M, cfg["IC"], cfg["OC"], cfg["K"])
    log("int8 prefill down 8192 x 17408 -> 5120")
    d = _dev_case(c)
    out = _run(c, d)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(5).choice(M, 6, replace=False)]))
    _sampled(c["x"], d["x"], [dict(c, col0=0)], [d], out, rows, 6)
