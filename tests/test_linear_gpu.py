"""GPU parity of the EXL3 linear layer against the fp64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import exl3_oracle as O
from moe_exl3_pre_amd import exl3, synth
from tests.helpers import (assert_close_linear, bf16_to_f64, dev, gpu_int8_codes, log, oracle_block_columns,
                           oracle_int8_block_columns, rel_fro, shard_to_dev, to_dev, to_dev_x)

pytestmark = pytest.mark.gpu

SENTINEL = -1000.0          # exactly representable in bf16


def _case_to_dev(c):
    return dict(x=to_dev_x(c["x_bits"]), code=to_dev(c["code"]), s_in=to_dev(c["s_in"]), rin=to_dev(c["rin"]),
                rout=to_dev(c["rout"]), s_out=to_dev(c["s_out"]))


def _run_linear(c, d, flags=0, ldo=None, col0=0, ws=None):
    M, OC = c["M"], c["OC"]
    ldo = ldo or OC
    out = torch.full((M, ldo), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_into(out, d["x"], d["code"], c["K"], d["s_in"], d["rin"], d["rout"], d["s_out"], col0=col0,
                     flags=flags, ws=ws)
    torch.cuda.synchronize()
    return out


# ------------------------------------------------------------------------------------------ decode

@pytest.mark.parametrize("K", range(1, 9))
def test_decode_tiles_bit_exact_all_k(K):
    log(f"decode_tiles K={K} IC=OC=128")
    rng = np.random.default_rng(200 + K)
    code = synth.random_code(rng, 128, 256, K)
    w = exl3.decode_tiles(to_dev(code), K).cpu().numpy()
    ref = O.decode_weight(code, K).astype(np.float16)
    assert np.array_equal(w.view(np.uint16), ref.view(np.uint16))


@pytest.mark.parametrize("IC,OC,K,rows", [(512, 512, 3, None), (4096, 14336, 2, 8), (4096, 14336, 3, 8),
                                          (5120, 17408, 2, 4), (17408, 5120, 3, 8), (2048, 768, 4, None)])
def test_decode_tiles_bit_exact_config_shapes(IC, OC, K, rows):
    log(f"decode_tiles IC={IC} OC={OC} K={K}")
    rng = np.random.default_rng(IC + OC + K)
    code = synth.random_code(rng, IC, OC, K)
    w = exl3.decode_tiles(to_dev(code), K)
    if rows is None:
        sel = np.arange(IC // 16)
    else:   # a sample of tile rows, always including the first and the last
        sel = np.unique(np.concatenate([[0, IC // 16 - 1], rng.choice(IC // 16, rows, replace=False)]))
    got = w.view(torch.int16).cpu().numpy().reshape(IC // 16, 16, OC)[sel].reshape(-1, OC)
    ref = O.decode_weight(code[sel], K).astype(np.float16).view(np.int16)
    assert np.array_equal(got, ref)


def test_decode_tiles_special_words():
    """All-zero words decode to 0.125 everywhere; all-ones words to 0.171875 (both sides of the wrap)."""
    for fill, val in ((0, 0.125), (-1, 0.171875)):
        for K in (2, 3, 4):
            code = np.full((4, 4, 16 * K), fill, dtype=np.int16)
            w = exl3.decode_tiles(to_dev(code), K).float().cpu().numpy()
            assert np.all(w == val)


# ------------------------------------------------------------------------------------------ pre-pass

def test_rotate_activations_fp16():
    c = synth.linear_case(1000, 5, 512, 128, 3)
    d = _case_to_dev(c)
    got = exl3.rotate_activations(d["x"], d["s_in"], d["rin"]).float().cpu().numpy()
    ref = O.rotate_input(c["x"], c["s_in"], c["rin"])
    ref16 = O.round_fp16(ref)
    # fp32 butterflies then one fp16 rounding: equal to the fp16 rounding of the exact value except at
    # near-ties, where it is the neighbouring fp16 number.
    diff = np.abs(got - ref16)
    ulp = np.abs(np.spacing(ref16.astype(np.float16))).astype(np.float64)
    assert np.all(diff <= ulp)
    assert np.mean(diff > 0) < 1e-3
    assert rel_fro(got, ref) < 2 ** -11


# ------------------------------------------------------------------------------------------ linear

def test_linear_small_config():
    """M=4, IC=OC=512, K=3: the whole output."""
    c = synth.linear_case(1000, **synth.SMALL)
    log("linear small config")
    out = _run_linear(c, _case_to_dev(c))
    got = bf16_to_f64(out)
    args = (c["code"], 3, c["s_in"], c["rin"], c["rout"], c["s_out"])
    e = assert_close_linear(got, O.linear(c["x"], *args, act="f16"), O.linear(c["x"], *args))
    log(f"  rel err {e:.3e}")


@pytest.mark.parametrize("M", [1, 2, 3, 5, 15, 16, 17, 33])
@pytest.mark.parametrize("K", [2, 3, 4])
def test_linear_ragged_m(M, K):
    log(f"linear ragged M={M} K={K}")
    c = synth.linear_case(3000 + 10 * M + K, M, 384, 256, K)
    out = _run_linear(c, _case_to_dev(c))
    args = (c["code"], K, c["s_in"], c["rin"], c["rout"], c["s_out"])
    assert_close_linear(bf16_to_f64(out), O.linear(c["x"], *args, act="f16"), O.linear(c["x"], *args))


@pytest.mark.parametrize("K", [1, 5, 6, 7, 8])
def test_linear_other_k(K):
    log(f"linear K={K}")
    c = synth.linear_case(4000 + K, 6, 256, 384, K)
    out = _run_linear(c, _case_to_dev(c))
    args = (c["code"], K, c["s_in"], c["rin"], c["rout"], c["s_out"])
    assert_close_linear(bf16_to_f64(out), O.linear(c["x"], *args, act="f16"), O.linear(c["x"], *args))


def test_linear_slice_leaves_other_columns():
    c = synth.linear_case(1001, 3, 256, 256, 2)
    out = _run_linear(c, _case_to_dev(c), ldo=640, col0=130)   # odd-aligned slice start (130 is even; ldo even)
    o = out.float().cpu().numpy()
    assert np.all(o[:, :130] == SENTINEL) and np.all(o[:, 386:] == SENTINEL)
    args = (c["code"], 2, c["s_in"], c["rin"], c["rout"], c["s_out"])
    assert_close_linear(o[:, 130:386].astype(np.float64), O.linear(c["x"], *args, act="f16"), O.linear(c["x"], *args))
    out2 = _run_linear(c, _case_to_dev(c), ldo=641, col0=131)  # 2-byte-aligned stores
    o2 = out2.float().cpu().numpy()
    assert np.array_equal(o2[:, 131:387], o[:, 130:386])
    assert np.all(o2[:, :131] == SENTINEL) and np.all(o2[:, 387:] == SENTINEL)


def test_linear_zero_rows_noop():
    c = synth.linear_case(1002, 0, 256, 256, 2)
    d = _case_to_dev(c)
    out = torch.full((0, 256), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_into(out, d["x"], d["code"], 2, d["s_in"], d["rin"], d["rout"], d["s_out"])


def test_linear_exact_symmetries():
    """s_in -> -s_in negates the output bit for bit; x -> 2x doubles it; zero input gives zeros."""
    c = synth.linear_case(1003, 4, 512, 256, 3)
    d = _case_to_dev(c)
    base = _run_linear(c, d)
    neg = _run_linear(c, dict(d, s_in=-d["s_in"]))
    assert torch.equal(neg, -base)
    dbl = _run_linear(c, dict(d, x=d["x"] * 2))
    assert torch.equal(dbl, base * 2)
    zero = _run_linear(c, dict(d, x=torch.zeros_like(d["x"])))
    assert torch.count_nonzero(zero.float()) == 0


def test_linear_rin_rout_not_interchangeable():
    c = synth.linear_case(1004, 4, 256, 256, 2)
    d = _case_to_dev(c)
    a = _run_linear(c, d)
    b = _run_linear(c, dict(d, rin=d["rout"], rout=d["rin"]))
    assert rel_fro(bf16_to_f64(b), bf16_to_f64(a)) > 1e-2


def test_linear_workspace_poison_counters_and_determinism():
    """Workspace filled with NaN bytes (except the zeroed counter head) gives the same bits; calls
    back to back without re-zeroing (the kernels reset their counters) give the same bits."""
    c = synth.linear_case(1005, 8, 1024, 1024, 3)
    d = _case_to_dev(c)
    nbytes = exl3.linear_workspace_bytes(8, 1024, 1024)
    ws = exl3.alloc_workspace(nbytes, dev())
    ref = _run_linear(c, d, ws=ws)
    for _ in range(3):
        again = _run_linear(c, d, ws=ws)
        assert torch.equal(again, ref)
    poisoned = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=dev())
    poisoned[:16384] = 0
    got = _run_linear(c, d, ws=poisoned)
    assert torch.equal(got, ref)


def test_linear_batch_invariance_decode_rows():
    """A row's output does not depend on the other rows of the batch (decode-phase kernel), also across
    the switch from in-block rotation (M <= 4) to activations rotated once per call (M >= 5) and across
    launches of one and of two 16-row groups (17..32 rows): M=48 runs as launches of 32 and 16 rows."""
    c = synth.linear_case(1006, 48, 512, 384, 2)
    d = _case_to_dev(c)
    assert exl3.lib().exl3_gemv_max_rows(384) >= 48
    full = _run_linear(c, d)
    for M in (1, 4, 5, 9, 16, 17, 32, 33, 36):
        sub = dict(c, M=M)
        part = _run_linear(sub, dict(d, x=d["x"][:M].contiguous()))
        assert torch.equal(part, full[:M])


@pytest.mark.parametrize("int8", [False, True])
def test_batch_invariant_flag_across_the_crossover(int8):
    """EXL3_BATCH_INVARIANT: at M in {1, 8, 16, 17, 32, 33, 48, 64, 300} a row's bits equal the bits of that
    row computed alone (M=1), although the default dispatch for this 5120-column shard switches to the
    GEMM above 32 rows (and its split count changes with M).  The 16-bit path runs the decode-phase
    kernel (launches of 32 rows and a remainder); the 8-bit path the unsplit GEMM.  The M=300 output
    meets the oracle on sampled column blocks (the 8-bit path on the kernel's own codes)."""
    IC, OC, K, MMAX = 512, 5120, 3, 300
    c = synth.linear_case(1011, MMAX, IC, OC, K)
    d = _case_to_dev(c)
    assert exl3.lib().exl3_gemv_max_rows(OC) == 32
    flags = exl3.BATCH_INVARIANT | (exl3.ACT_INT8 if int8 else 0)
    full = _run_linear(c, d, flags=flags)
    for r in list(range(0, MMAX, 13)) + [MMAX - 1]:
        one = _run_linear(dict(c, M=1), dict(d, x=d["x"][r:r + 1].contiguous()), flags=flags)
        assert torch.equal(one[0], full[r]), r
    for M in (1, 8, 16, 17, 32, 33, 48, 64):
        part = _run_linear(dict(c, M=M), dict(d, x=d["x"][:M].contiguous()), flags=flags)
        assert torch.equal(part, full[:M]), M
    blocks = [0, OC // 128 - 1, 17]
    got = bf16_to_f64(full)
    if int8:
        q, sc = gpu_int8_codes(d["x"], d["s_in"], d["rin"], c["x"], c["s_in"], c["rin"])
        cols, y8 = oracle_int8_block_columns(q, sc, c["code"], K, c["rout"], c["s_out"], blocks)
        _, y64 = oracle_block_columns(c["x"], c["code"], K, c["s_in"], c["rin"], c["rout"], c["s_out"], blocks)
        assert_close_linear(got[:, cols], y8, y64, tol=3e-2)
    else:
        args = (c["x"], c["code"], K, c["s_in"], c["rin"], c["rout"], c["s_out"], blocks)
        cols, y64 = oracle_block_columns(*args)
        _, y16 = oracle_block_columns(*args, act="f16")
        assert_close_linear(got[:, cols], y16, y64)


# ------------------------------------------------------------------------------------------ merged shards

@pytest.mark.parametrize("M", [1, 2, 4, 8, 24])
def test_decode_gate_up_config(M):
    """Merged gate (K=2) | up (K=3), IC=4096, 2 x 14336 columns: multi-shard call == per-shard calls
    bit for bit, and sampled 128-column blocks of both shards match the oracle."""
    cfg = synth.DECODE_GATE_UP
    case = synth.merged_case(1100 + M, M, cfg["IC"], [(cfg["OC_gate"], cfg["K_gate"]), (cfg["OC_up"], cfg["K_up"])])
    log(f"gate_up decode M={M}")
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    shards = [shard_to_dev(s, s_in, rin) for s in case["shards"]]
    out = torch.full((M, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(out, x, shards)
    out2 = torch.full_like(out, SENTINEL)
    for s in shards:
        exl3.linear_into(out2, x, s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], col0=s["col0"])
    torch.cuda.synchronize()
    assert torch.equal(out, out2)
    got = bf16_to_f64(out)
    rng = np.random.default_rng(M)
    for s in case["shards"]:
        blocks = sorted(set([0, s["OC"] // 128 - 1] + list(rng.choice(s["OC"] // 128, 3, replace=False))))
        cols, y64 = oracle_block_columns(case["x"], s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], blocks)
        _, y16 = oracle_block_columns(case["x"], s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"], blocks,
                                      act="f16")
        e = assert_close_linear(got[:, s["col0"] + cols], y16, y64)
        log(f"  shard K={s['K']} rel err {e:.3e}")


def test_merged_shards_with_distinct_input_vectors():
    case = synth.merged_case(1200, 5, 512, [(256, 2), (384, 3), (128, 4)], shared_input_vectors=False)
    x = to_dev_x(case["x_bits"])
    shards = [shard_to_dev(s) for s in case["shards"]]
    out = torch.full((5, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(out, x, shards)
    torch.cuda.synchronize()
    got = bf16_to_f64(out)
    for s in case["shards"]:
        args = (s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"])
        assert_close_linear(got[:, s["col0"]:s["col0"] + s["OC"]], O.linear(case["x"], *args, act="f16"),
                            O.linear(case["x"], *args))


@pytest.mark.parametrize("M", [3, 8, 24, 40])
def test_large_ic_sampled(M):
    """down_proj shape IC=17408, OC=5120, K=3 at decode M (many splits), sampled blocks; M=8 takes the
    activations rotated once per call (a 16 x 17408 fragment-major region of the workspace), M=24 one
    launch of two 16-row groups, M=40 launches of 32 and 8 rows."""
    c = synth.linear_case(1300 + M, M, 17408, 5120, 3)
    log(f"large IC sampled M={M}")
    out = _run_linear(c, _case_to_dev(c))
    got = bf16_to_f64(out)
    blocks = [0, 17, 39]
    cols, y64 = oracle_block_columns(c["x"], c["code"], 3, c["s_in"], c["rin"], c["rout"], c["s_out"], blocks)
    _, y16 = oracle_block_columns(c["x"], c["code"], 3, c["s_in"], c["rin"], c["rout"], c["s_out"], blocks, act="f16")
    assert_close_linear(got[:, cols], y16, y64)


# ------------------------------------------------------------------------------------------ graph capture

@pytest.mark.parametrize("M", [4, 8])
def test_graph_capture_replay_matches_eager(M):
    """M=4 rotates in every block; M=8 adds the once-per-call rotation launch before the decode kernel."""
    cfg = synth.DECODE_GATE_UP
    log(f"graph capture M={M}")
    case = synth.merged_case(1400 + M, M, 1024, [(512, 2), (768, 3)])
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    shards = [shard_to_dev(s, s_in, rin) for s in case["shards"]]
    ws = exl3.alloc_workspace(exl3.linear_multi_workspace_bytes(M, 1024, shards), dev())
    eager = torch.zeros((M, case["ldo"]), dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(eager, x, shards, ws=ws)
    torch.cuda.synchronize()
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        exl3.linear_multi_into(out, x, shards, ws=ws)      # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        exl3.linear_multi_into(out, x, shards, ws=ws)
    for i in range(4):
        out.fill_(float(i))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        tmp = torch.zeros_like(eager)                        # eager work between replays
        exl3.linear_multi_into(tmp, x, shards, ws=ws)
        torch.cuda.synchronize()
        assert torch.equal(tmp, eager)
    del cfg
