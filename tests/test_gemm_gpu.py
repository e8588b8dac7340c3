"""GPU parity of the prefill-phase (MFMA GEMM) path against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import exl3_oracle as O
from moe_exl3_pre_amd import exl3, synth
from tests.helpers import (assert_close_linear, bf16_to_f64, dev, gpu_int8_codes, log, oracle_block_columns,
                           oracle_int8_block_columns, rel_fro, shard_to_dev, to_dev, to_dev_x)

pytestmark = pytest.mark.gpu

SENTINEL = -1000.0


def _dev_case(c):
    return dict(x=to_dev_x(c["x_bits"]), code=to_dev(c["code"]), s_in=to_dev(c["s_in"]), rin=to_dev(c["rin"]),
                rout=to_dev(c["rout"]), s_out=to_dev(c["s_out"]))


def _run(c, d, flags, ldo=None, col0=0):
    out = torch.full((c["M"], ldo or c["OC"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_into(out, d["x"], d["code"], c["K"], d["s_in"], d["rin"], d["rout"], d["s_out"], col0=col0, flags=flags)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("M", [1, 3, 17, 64, 255, 300])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_mfma_path_ragged(M, K):
    log(f"mfma ragged M={M} K={K}")
    c = synth.linear_case(5000 + 7 * M + K, M, 384, 384, K)      # 3 column blocks: one odd 128-column tile
    out = _run(c, _dev_case(c), exl3.FORCE_MFMA)
    args = (c["code"], K, c["s_in"], c["rin"], c["rout"], c["s_out"])
    assert_close_linear(bf16_to_f64(out), O.linear(c["x"], *args, act="f16"), O.linear(c["x"], *args))


@pytest.mark.parametrize("K", [1, 5, 6, 7, 8])
def test_mfma_path_other_k(K):
    c = synth.linear_case(5100 + K, 40, 256, 256, K)
    out = _run(c, _dev_case(c), exl3.FORCE_MFMA)
    args = (c["code"], K, c["s_in"], c["rin"], c["rout"], c["s_out"])
    assert_close_linear(bf16_to_f64(out), O.linear(c["x"], *args, act="f16"), O.linear(c["x"], *args))


def test_default_dispatch_uses_mfma_above_threshold():
    """Above exl3_gemv_max_rows(OC) the default call equals the forced MFMA call bit for bit; at or below
    it equals the forced decode-phase call."""
    thr = exl3.lib().exl3_gemv_max_rows(256)
    for M, force in ((thr, exl3.FORCE_GEMV), (thr + 1, exl3.FORCE_MFMA), (200, exl3.FORCE_MFMA)):
        c = synth.linear_case(5200 + M, M, 512, 256, 3)
        d = _dev_case(c)
        assert torch.equal(_run(c, d, 0), _run(c, d, force)), M


def test_decode_and_mfma_paths_agree():
    c = synth.linear_case(5300, 48, 1024, 512, 3)
    d = _dev_case(c)
    a = bf16_to_f64(_run(c, d, exl3.FORCE_GEMV))
    b = bf16_to_f64(_run(c, d, exl3.FORCE_MFMA))
    assert rel_fro(a, b) < 4e-3
    args = (c["code"], 3, c["s_in"], c["rin"], c["rout"], c["s_out"])
    ref16 = O.linear(c["x"], *args, act="f16")
    ref = O.linear(c["x"], *args)
    assert_close_linear(a, ref16, ref)
    assert_close_linear(b, ref16, ref)


def test_mfma_slice_and_sentinel():
    c = synth.linear_case(5400, 70, 256, 256, 2)
    out = _run(c, _dev_case(c), exl3.FORCE_MFMA, ldo=640, col0=256)
    o = out.float().cpu().numpy()
    assert np.all(o[:, :256] == SENTINEL) and np.all(o[:, 512:] == SENTINEL)
    args = (c["code"], 2, c["s_in"], c["rin"], c["rout"], c["s_out"])
    assert_close_linear(o[:, 256:512].astype(np.float64), O.linear(c["x"], *args, act="f16"), O.linear(c["x"], *args))


def test_mfma_exact_symmetries_and_determinism():
    c = synth.linear_case(5500, 130, 512, 384, 3)
    d = _dev_case(c)
    base = _run(c, d, exl3.FORCE_MFMA)
    assert torch.equal(_run(c, d, exl3.FORCE_MFMA), base)
    assert torch.equal(_run(c, dict(d, s_in=-d["s_in"]), exl3.FORCE_MFMA), -base)


def test_mfma_batch_invariance():
    """Without the feature split a row's output does not depend on the other rows (each output element is
    one fixed-order reduction), so a prefix of the batch reproduces the same rows."""
    c = synth.linear_case(5600, 300, 1024, 256, 2)
    d = _dev_case(c)
    flags = exl3.FORCE_MFMA | exl3.GEMM_NO_SPLIT
    full = _run(c, d, flags)
    assert exl3.lib().exl3_gemm_splits(77, 1024, 256) > 1     # the split would change the rounding
    for M in (1, 77, 256):
        part = _run(dict(c, M=M), dict(d, x=d["x"][:M].contiguous()), flags)
        assert torch.equal(part, full[:M]), M


def _sampled_check(case_x, shards, out, rows, blocks_per_shard=3, seed=0):
    got = bf16_to_f64(out)[rows]
    rng = np.random.default_rng(seed)
    x = case_x[rows]
    for s in shards:
        nblk = s["OC"] // 128
        blocks = sorted(set([0, nblk - 1] + list(rng.choice(nblk, blocks_per_shard, replace=False))))
        cols, y64 = oracle_block_columns(x, s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], blocks)
        _, y16 = oracle_block_columns(x, s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], blocks,
                                      act="f16")
        e = assert_close_linear(got[:, s["col0"] + cols], y16, y64)
        log(f"  shard K={s['K']} OC={s['OC']}: rel err {e:.3e} on {len(rows)} rows x {len(cols)} cols")


def test_prefill_gate_up_full_size_sampled():
    """M=8192, IC=5120, gate (K=2) | up (K=3) of 17408 columns each: full-size run, sampled check."""
    p = synth.PREFILL
    cfg = p["gate_up"]
    M = p["M"]
    case = synth.merged_case(2000, M, cfg["IC"], [(cfg["OC"], cfg["K_gate"]), (cfg["OC"], cfg["K_up"])])
    log("prefill gate_up 8192 x 5120 -> 2 x 17408")
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    shards = [shard_to_dev(s, s_in, rin) for s in case["shards"]]
    out = torch.full((M, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(out, x, shards)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(1).choice(M, 12, replace=False)]))
    _sampled_check(case["x"], case["shards"], out, rows)


def test_prefill_down_full_size_sampled():
    p = synth.PREFILL
    cfg = p["down"]
    M = p["M"]
    c = synth.linear_case(2001, M, cfg["IC"], cfg["OC"], cfg["K"])
    log("prefill down 8192 x 17408 -> 5120")
    out = _run(c, _dev_case(c), 0)
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(2).choice(M, 10, replace=False)]))
    _sampled_check(c["x"], [dict(c, col0=0)], out, rows)


def test_tail_round_split_parity():
    """A shard whose 4-wave blocks leave the last round at most half full runs that round's blocks with
    their input features split (exl3_gemm_tail_splits).  Here 9 x 29 = 261 blocks: the last 5 are row
    tile 8 x column tiles 96..115.  All rows of 7 column blocks (4 inside that region) against the
    oracle on the 16-bit and the 8-bit path; only tiles of that region differ from the unsplit GEMM, and
    repeated calls give the same bits."""
    M, IC, OC, K = 1152, 1024, 14848, 3
    L = exl3.lib()
    assert L.exl3_gemm_splits(M, IC, OC) == 1 and L.exl3_gemm_tail_splits(M, IC, OC) == 2
    log(f"tail-round split M={M} IC={IC} OC={OC} K={K}")
    c = synth.linear_case(5950, M, IC, OC, K)
    d = _dev_case(c)
    blocks = [0, 47, 95, 96, 103, 110, 115]
    args = (c["x"], c["code"], K, c["s_in"], c["rin"], c["rout"], c["s_out"], blocks)
    cols, y64 = oracle_block_columns(*args)
    out = _run(c, d, 0)
    assert_close_linear(bf16_to_f64(out)[:, cols], oracle_block_columns(*args, act="f16")[1], y64)
    assert torch.equal(_run(c, d, 0), out)
    ref = _run(c, d, exl3.GEMM_NO_SPLIT)
    differ = (out != ref).view(M // 128, 128, OC // 128, 128).any(dim=3).any(dim=1).cpu().numpy()
    mt, ct = np.nonzero(differ)
    assert np.all(mt == 8) and np.all(ct >= 96), (mt, ct)
    # 8-bit path: the oracle's contraction on the kernel's own codes (checked against the oracle's
    # quantisation first), every element at the same bar
    got8 = bf16_to_f64(_run(c, d, exl3.ACT_INT8))[:, cols]
    q, sc = gpu_int8_codes(d["x"], d["s_in"], d["rin"], c["x"], c["s_in"], c["rin"])
    _, y8 = oracle_int8_block_columns(q, sc, c["code"], K, c["rout"], c["s_out"], blocks)
    assert_close_linear(got8, y8, y64, tol=3e-2)


def test_tail_round_split_poisoned_workspace():
    """The split tail's partial tiles are written before they are read: a workspace filled with NaN bytes
    (the counter head zeroed, as the ABI asks once) gives the same bits as a zeroed one."""
    M, IC, OC, K = 1152, 1024, 14848, 2
    c = synth.linear_case(5970, M, IC, OC, K)
    d = _dev_case(c)
    nbytes = exl3.linear_workspace_bytes(M, IC, OC)
    outs = []
    for fill in (0x00, 0xFF):
        ws = torch.full((nbytes,), fill, dtype=torch.uint8, device=dev())
        ws[:16384] = 0
        out = torch.full((M, OC), SENTINEL, dtype=torch.bfloat16, device=dev())
        exl3.linear_into(out, d["x"], d["code"], K, d["s_in"], d["rin"], d["rout"], d["s_out"], ws=ws)
        torch.cuda.synchronize()
        outs.append(out)
    assert torch.isfinite(outs[1].float()).all()
    assert torch.equal(outs[0], outs[1])


def test_tail_round_split_merged_equals_separate():
    """Two shards that each split their tail round (K=2 | K=3, 261 blocks apiece): the merged call equals
    one call per shard bit for bit (each shard's plan depends only on its own M, IC, OC)."""
    M, IC, OC = 1152, 1024, 14848
    assert exl3.lib().exl3_gemm_tail_splits(M, IC, OC) == 2
    case = synth.merged_case(5960, M, IC, [(OC, 2), (OC, 3)])
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    shards = [shard_to_dev(s, s_in, rin) for s in case["shards"]]
    merged = torch.full((M, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(merged, x, shards)
    sep = torch.full_like(merged, SENTINEL)
    for s in shards:
        exl3.linear_into(sep, x, s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], col0=s["col0"])
    torch.cuda.synchronize()
    assert torch.equal(merged, sep)


# ------------------------------------------------------------------ K-split GEMM (default flags, small M)

@pytest.mark.parametrize("M,IC,OC,K", [(200, 2048, 256, 2), (300, 1536, 384, 3), (131, 4096, 128, 4)])
def test_split_k_parity(M, IC, OC, K):
    """Above the decode-phase threshold but with few output tiles the GEMM splits the input features;
    the split partial tiles summed in order match the oracle like the unsplit GEMM."""
    splits = exl3.lib().exl3_gemm_splits(M, IC, OC)
    assert splits > 1 and M > exl3.lib().exl3_gemv_max_rows(OC)
    log(f"split-K M={M} IC={IC} OC={OC} K={K}: {splits} splits")
    c = synth.linear_case(5700 + M + K, M, IC, OC, K)
    d = _dev_case(c)
    out = _run(c, d, 0)
    args = (c["code"], K, c["s_in"], c["rin"], c["rout"], c["s_out"])
    assert_close_linear(bf16_to_f64(out), O.linear(c["x"], *args, act="f16"), O.linear(c["x"], *args))
    assert torch.equal(_run(c, d, 0), out)                    # fixed summation order: deterministic
    unsplit = bf16_to_f64(_run(c, d, exl3.FORCE_MFMA | exl3.GEMM_NO_SPLIT))
    assert rel_fro(bf16_to_f64(out), unsplit) < 1e-2


def test_split_k_int8_small_m():
    M, IC, OC = 20, 2048, 256
    assert exl3.lib().exl3_gemm_splits(M, IC, OC) > 1
    c = synth.linear_case(5800, M, IC, OC, 3)
    d = _dev_case(c)
    out = _run(c, d, exl3.ACT_INT8)
    args = (c["code"], 3, c["s_in"], c["rin"], c["rout"], c["s_out"])
    q, sc = gpu_int8_codes(d["x"], d["s_in"], d["rin"], c["x"], c["s_in"], c["rin"])
    assert_close_linear(bf16_to_f64(out), O.linear_from_int8(q, sc, c["code"], 3, c["rout"], c["s_out"]),
                        O.linear(c["x"], *args), tol=3e-2)


def test_split_k_down_full_width_sampled():
    """M=200 rows of the 17408 -> 5120 down projection (K=3): 80 tiles, the features split in many."""
    cfg = synth.PREFILL["down"]
    M = 200
    assert exl3.lib().exl3_gemm_splits(M, cfg["IC"], cfg["OC"]) > 4
    c = synth.linear_case(2002, M, cfg["IC"], cfg["OC"], cfg["K"])
    out = _run(c, _dev_case(c), 0)
    rows = np.array([0, 77, 128, 199])
    _sampled_check(c["x"], [dict(c, col0=0)], out, rows)


def _merged_dev(case):
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    return x, [shard_to_dev(s, s_in, rin) for s in case["shards"]]


def test_split_k_merged_equals_separate():
    """Shards with different split plans in one call: each shard's split depends only on (M, IC, OC), so
    the merged call equals one call per shard bit for bit (the slab is shared, the shards run in turn)."""
    M, IC = 200, 1024
    case = synth.merged_case(5900, M, IC, [(256, 2), (384, 3), (128, 4)])
    plans = [exl3.lib().exl3_gemm_splits(M, IC, s["OC"]) for s in case["shards"]]
    assert all(p > 1 for p in plans) and M > exl3.lib().exl3_gemv_max_rows(384)
    x, shards = _merged_dev(case)
    merged = torch.full((M, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(merged, x, shards)
    sep = torch.full_like(merged, SENTINEL)
    for s in shards:
        exl3.linear_multi_into(sep, x, [s])
    torch.cuda.synchronize()
    assert torch.equal(merged, sep)
    _sampled_check(case["x"], case["shards"], merged, np.arange(0, M, 17), blocks_per_shard=1)


def test_split_k_graph_replay_matches_eager():
    """The split path (GEMM launch + reduction launch, no memset) captured in a graph and replayed with eager
    work between the replays."""
    M, IC = 150, 2048
    case = synth.merged_case(5901, M, IC, [(256, 3)])
    assert exl3.lib().exl3_gemm_splits(M, IC, 256) > 1
    x, shards = _merged_dev(case)
    ws = exl3.alloc_workspace(exl3.linear_multi_workspace_bytes(M, IC, shards), dev())
    eager = torch.zeros((M, case["ldo"]), dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(eager, x, shards, ws=ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        exl3.linear_multi_into(out, x, shards, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        exl3.linear_multi_into(out, x, shards, ws=ws)
    for i in range(3):
        out.fill_(float(i))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        tmp = torch.zeros_like(eager)
        exl3.linear_multi_into(tmp, x, shards, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(tmp, eager)


# ------------------------------------------------------------------ the 64-layer sweep's projections

@pytest.mark.parametrize("M", [64, 512])
@pytest.mark.parametrize("name,IC,OC,K", [("qkv", 5120, 7168, 3), ("o", 5120, 5120, 3)])
def test_sweep_projections_both_paths_sampled(name, IC, OC, K, M):
    """The decoder sweep's attention projections (hidden 5120: qkv 5120 -> 7168, o 5120 -> 5120, K=3) at the
    sweep's mid sizes, on the decode-phase path (16-row launches) and on the MFMA GEMM: every row of five
    128-column blocks (the first, the last and three at random) against the oracle."""
    c = synth.linear_case(7000 + OC // 128 + M, M, IC, OC, K)
    d = _dev_case(c)
    rows = np.arange(M)
    for tag, flags in (("decode", exl3.FORCE_GEMV), ("mfma", exl3.FORCE_MFMA)):
        log(f"{name} {IC}->{OC} K={K} M={M} on the {tag} path")
        out = _run(c, d, flags)
        _sampled_check(c["x"], [dict(c, col0=0)], out, rows, seed=M)
