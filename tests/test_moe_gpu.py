"""GPU parity of the MoE expert-bank forward against the fp64 oracle's dense per-expert loop, through
the C ABI."""
import ctypes

import numpy as np
import pytest
import torch

from oracle import exl3_oracle as O
from moe_exl3_pre_amd import exl3, synth
from moe_exl3_pre_amd.bank import DeviceBank, pack_bank
from tests.helpers import assert_close_linear, bf16_to_f64, dev, log, to_dev, to_dev_x

pytestmark = pytest.mark.gpu


def _setup(m):
    bank = DeviceBank(pack_bank(m["experts"], m["H"], m["I"]), dev())
    x = to_dev_x(m["x_bits"])
    ids = to_dev(m["topk_ids"].astype(np.int32))
    w = to_dev(m["topk_w"].astype(np.float32))
    return bank, x, ids, w


# the two plans: the decode-sized one (32-row chunks, streaming core) and the prefill one (64-row
# chunks, grouped 64 x 128 tiles); by default the call picks one by the pairs per expert
PLANS = {"decode_plan": exl3.FORCE_GEMV, "prefill_plan": exl3.FORCE_MFMA}


def _run(bank, x, ids, w, ws=None, flags=0):
    out = torch.full(x.shape, -1000.0, dtype=torch.bfloat16, device=dev())
    exl3.moe_bank_forward(out, x, ids, w, bank, ws=ws, flags=flags)
    torch.cuda.synchronize()
    return out


def _check(m, out, tokens=None, experts=None):
    ex = m["experts"] if experts is None else experts
    ref = O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], ex, tokens=tokens)
    ref16 = O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], ex, act="f16", tokens=tokens)
    got = bf16_to_f64(out)
    rows = np.arange(m["T"]) if tokens is None else np.asarray(tokens)
    e = assert_close_linear(got[rows], ref16[rows], ref[rows])
    log(f"  rel err {e:.3e} over {len(rows)} tokens")
    return e


@pytest.mark.parametrize("cfg", [
    dict(T=64, E=16, topk=4, H=256, I=256, Ks=(2, 3, 4)),                        # one mixed-K launch
    dict(T=48, E=12, topk=3, H=256, I=384, Ks=(2, 3, 4), k_d_independent=True),  # k_gu != k_d
    dict(T=40, E=8, topk=2, H=384, I=128, Ks=(1, 5)),                            # one launch per K; odd H blocks
    dict(T=56, E=12, topk=3, H=256, I=256, Ks=(6, 7, 8), k_d_independent=True),  # the widest codes, per-K launches
    dict(T=1, E=8, topk=8, H=256, I=128, Ks=(2, 3, 4)),                          # one token, every expert
])
@pytest.mark.parametrize("plan", list(PLANS))
def test_moe_small_full_parity(cfg, plan):
    cfg = dict(cfg)
    log(f"moe parity {cfg} {plan}")
    m = synth.moe_case(700 + cfg["T"], **cfg)
    # every K of the case is present in both projections, so each per-K kernel runs
    for key in ("k_gu", "k_d"):
        assert {e[key] for e in m["experts"]} == set(cfg["Ks"])
    bank, x, ids, w = _setup(m)
    _check(m, _run(bank, x, ids, w, flags=PLANS[plan]))


@pytest.mark.parametrize("plan", list(PLANS))
def test_moe_many_rows_per_expert_and_empty_expert(plan):
    """~100 rows per expert (several 32-row chunks, one partial; a full and a partial 64-row chunk on the
    prefill plan) and one expert with no token."""
    m = synth.moe_case(711, T=200, E=5, topk=2, H=256, I=256, Ks=(2, 3, 4))
    rng = np.random.default_rng(9)
    ids = np.stack([rng.choice(4, 2, replace=False) for _ in range(m["T"])]).astype(np.int32)   # expert 4 unused
    m = dict(m, topk_ids=ids)
    log(f"moe many rows: counts {np.bincount(ids.ravel(), minlength=5)} {plan}")
    bank, x, dids, w = _setup(m)
    _check(m, _run(bank, x, dids, w, flags=PLANS[plan]))


@pytest.mark.parametrize("T,E,topk", [(2048, 64, 4), (4608, 32, 4), (4096, 128, 8)])
def test_moe_route_counting_sort_path(T, E, topk):
    """Prefill-sized routing: E * ceil(T * topk / 32) exceeds the bitmap route's 8192 LDS words, so the
    counting-sort route runs -- with its LDS cache of the pairs' slots (8192 pairs) and without it
    (18432 pairs; 32,768 pairs over 128 experts, the prefill-sized bank's routing).  Sampled tokens against
    the oracle; a second call gives the same bits."""
    P = T * topk
    assert E * ((P + 31) // 32) > 8192
    log(f"moe counting-sort route T={T} E={E} top-{topk} ({P} pairs)")
    m = synth.moe_case(730 + E, T=T, E=E, topk=topk, H=256, I=128, Ks=(2, 3, 4))
    bank, x, ids, w = _setup(m)
    out = _run(bank, x, ids, w)
    assert torch.isfinite(out.float()).all()
    rng = np.random.default_rng(T)
    tokens = sorted(set([0, 1, T // 2, T - 1] + list(rng.choice(T, 12, replace=False))))
    _check(m, out, tokens=tokens)
    assert torch.equal(_run(bank, x, ids, w), out)


@pytest.mark.parametrize("plan", list(PLANS))
def test_moe_out_of_range_ids_are_ignored(plan):
    f = PLANS[plan]
    m = synth.moe_case(712, T=32, E=8, topk=4, H=256, I=128)
    ids = m["topk_ids"].copy()
    ids[3, 2] = -1
    ids[9, 0] = 8
    ids[17, 3] = 1 << 30
    m_bad = dict(m, topk_ids=ids)
    bank, x, dids, w = _setup(m_bad)
    out_bad = _run(bank, x, dids, w, flags=f)
    _check(m_bad, out_bad)
    # same as routing those terms to a real expert with weight zero (rows are independent, so bitwise)
    ids0 = m["topk_ids"].copy()
    w0 = m["topk_w"].copy()
    for t, j in ((3, 2), (9, 0), (17, 3)):
        w0[t, j] = 0.0
    out0 = _run(bank, x, to_dev(ids0.astype(np.int32)), to_dev(w0.astype(np.float32)), flags=f)
    assert torch.equal(out_bad, out0)


@pytest.mark.parametrize("plan", list(PLANS))
def test_moe_every_id_dropped_gives_zeros(plan):
    """No pair reaches an expert (ids negative or >= E): the route yields no chunk, the expert launches find
    no work, and every output element is an exact zero, as in the oracle's per-expert loop."""
    m = synth.moe_case(716, T=24, E=8, topk=3, H=256, I=128)
    ids = np.full_like(m["topk_ids"], -1)
    ids[::2, 1] = m["E"]
    ids[1::3, 2] = 1 << 20
    m_bad = dict(m, topk_ids=ids)
    log(f"moe all ids dropped {plan}")
    bank, x, dids, w = _setup(m_bad)
    out = _run(bank, x, dids, w, flags=PLANS[plan])
    assert torch.equal(out, torch.zeros_like(out))
    assert not np.any(O.moe_forward(m_bad["x"], ids, m_bad["topk_w"], m_bad["experts"]))


def test_moe_zero_tokens_is_a_no_op():
    """T = 0 through the C ABI returns OK and leaves the output buffer untouched."""
    m = synth.moe_case(717, T=4, E=8, topk=2, H=256, I=128)
    bank, x, ids, w = _setup(m)
    out = torch.full(x.shape, -1000.0, dtype=torch.bfloat16, device=dev())
    ws = exl3.alloc_workspace(exl3.moe_workspace_bytes(bank, 4, 2), dev())
    rc = exl3.lib().exl3_moe_bank_forward(exl3._ptr(out), exl3._ptr(x), 0, exl3._ptr(ids), exl3._ptr(w), 2,
                                           ctypes.byref(bank.struct), 0, exl3._ptr(ws), ws.numel(),
                                           exl3._stream(dev()))
    torch.cuda.synchronize()
    assert rc == exl3.OK
    assert torch.equal(out, torch.full_like(out, -1000.0))


@pytest.mark.parametrize("plan", list(PLANS))
def test_moe_deterministic_and_relabel_invariant(plan):
    f = PLANS[plan]
    m = synth.moe_case(713, T=64, E=16, topk=4, H=256, I=256)
    bank, x, ids, w = _setup(m)
    a = _run(bank, x, ids, w, flags=f)
    assert torch.equal(_run(bank, x, ids, w, flags=f), a)
    # relabel the logical experts: the packed slots and every pair's computation are unchanged
    perm = np.random.default_rng(5).permutation(m["E"])
    experts2 = [None] * m["E"]
    for e in range(m["E"]):
        experts2[perm[e]] = m["experts"][e]
    m2 = dict(m, experts=experts2, topk_ids=perm[m["topk_ids"]].astype(np.int32))
    bank2, x2, ids2, w2 = _setup(m2)
    b = _run(bank2, x2, ids2, w2, flags=f)
    # slots are a stable sort by K, so relabeling can reorder slots inside a group; rows are independent
    # and every reduction is fixed-order, so the result is still bit-identical
    assert torch.equal(a, b)


def test_moe_workspace_reuse_with_fewer_tokens():
    m = synth.moe_case(714, T=96, E=8, topk=2, H=256, I=128)
    bank, x, ids, w = _setup(m)
    ws = exl3.alloc_workspace(exl3.moe_workspace_bytes(bank, 96, 2), dev())
    full = _run(bank, x, ids, w, ws=ws)
    assert torch.equal(_run(bank, x, ids, w), full)
    part = _run(bank, x[:40].contiguous(), ids[:40].contiguous(), w[:40].contiguous(), ws=ws)
    assert torch.equal(part, full[:40])


def test_moe_graph_replay_matches_eager():
    m = synth.moe_case(715, T=32, E=8, topk=2, H=256, I=128)
    bank, x, ids, w = _setup(m)
    ws = exl3.alloc_workspace(exl3.moe_workspace_bytes(bank, 32, 2), dev())
    eager = _run(bank, x, ids, w, ws=ws)
    out = torch.zeros_like(eager)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        exl3.moe_bank_forward(out, x, ids, w, bank, ws=ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        exl3.moe_bank_forward(out, x, ids, w, bank, ws=ws)
    for i in range(3):
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), i
        _run(bank, x, ids, w, ws=ws)          # eager work between replays


def _full_size_tokens(m, n=32, seed=0):
    """At least n tokens that together route to every K group, to the most-loaded expert and to the
    least-loaded expert that has any token; the rest drawn at random."""
    ids = m["topk_ids"]
    load = np.bincount(ids.ravel(), minlength=m["E"])
    used = np.nonzero(load)[0]
    e_max, e_min = int(used[np.argmax(load[used])]), int(used[np.argmin(load[used])])
    pick = set()
    for e in (e_max, e_min):
        pick.update(np.nonzero((ids == e).any(axis=1))[0][:2].tolist())
    ks = np.array([m["experts"][e]["k_gu"] for e in range(m["E"])])
    for K in np.unique(ks):
        pick.update(np.nonzero((ks[ids] == K).any(axis=1))[0][:1].tolist())
    rng = np.random.default_rng(seed)
    rest = [t for t in rng.permutation(m["T"]) if t not in pick]
    pick.update(rest[:max(0, n - len(pick))])
    tokens = sorted(pick)
    assert e_max in ids[tokens] and e_min in ids[tokens]
    assert set(ks[ids[tokens]].ravel()) == set(np.unique(ks))
    return tokens, e_max, e_min


def test_moe_full_size_sampled():
    """T=256 tokens, 128 experts, top-8, H=2048, I=768, K in {2,3,4}: full run; 32 tokens (256 of the 2048
    (token, expert) pairs) checked element-wise, covering every K group and the most- and least-loaded
    experts; every other output finite."""
    cfg = synth.MOE
    m = synth.moe_case(1003, T=cfg["T"], E=cfg["E"], topk=cfg["topk"], H=cfg["H"], I=cfg["I"], Ks=cfg["Ks"])
    log("moe full size 256 x 2048, 128 experts top-8")
    bank, x, ids, w = _setup(m)
    out = _run(bank, x, ids, w)
    assert torch.isfinite(out.float()).all()
    tokens, e_max, e_min = _full_size_tokens(m)
    used = np.unique(m["topk_ids"][tokens])
    log(f"  {len(tokens)} tokens over {len(used)} experts (most loaded {e_max}, least loaded {e_min})")
    experts = list(m["experts"])
    for e in used:      # decode the touched experts once for both oracle variants
        d = experts[e]
        experts[e] = dict(d, W1=O.decode_weight(d["w1"], d["k_gu"]), W3=O.decode_weight(d["w3"], d["k_gu"]),
                          W2=O.decode_weight(d["w2"], d["k_d"]))
    _check(m, out, tokens=tokens, experts=experts)


def test_moe_plan_choice_by_pairs_per_expert():
    """Without a FORCE flag the call runs the decode-sized plan below 128 routed pairs per expert and the
    prefill plan from there on (bitwise the forced calls)."""
    for T, plan in ((254, "decode_plan"), (256, "prefill_plan")):      # 8 experts, top-4: 127 and 128 per expert
        m = synth.moe_case(740 + T, T=T, E=8, topk=4, H=256, I=128)
        bank, x, ids, w = _setup(m)
        assert torch.equal(_run(bank, x, ids, w), _run(bank, x, ids, w, flags=PLANS[plan])), T


def test_moe_prefill_bank_full_size_sampled():
    """The prefill-sized call on the full bank shape: T=4096 tokens, 128 experts, top-8 (32,768 pairs, ~256
    rows per expert: four or five 64-row chunks each), H=2048, I=768, K in {2,3,4}; 16 tokens against the oracle,
    covering every K group and the most- and least-loaded experts."""
    cfg = synth.MOE
    T = 4096
    m = synth.moe_case(1103, T=T, E=cfg["E"], topk=cfg["topk"], H=cfg["H"], I=cfg["I"], Ks=cfg["Ks"])
    log("moe prefill plan 4096 x 2048, 128 experts top-8")
    bank, x, ids, w = _setup(m)
    out = _run(bank, x, ids, w)
    assert torch.isfinite(out.float()).all()
    assert torch.equal(out, _run(bank, x, ids, w, flags=exl3.FORCE_MFMA))
    tokens, e_max, e_min = _full_size_tokens(m, n=16, seed=3)
    used = np.unique(m["topk_ids"][tokens])
    log(f"  {len(tokens)} tokens over {len(used)} experts")
    experts = list(m["experts"])
    for e in used:
        d = experts[e]
        experts[e] = dict(d, W1=O.decode_weight(d["w1"], d["k_gu"]), W3=O.decode_weight(d["w3"], d["k_gu"]),
                          W2=O.decode_weight(d["w2"], d["k_d"]))
    _check(m, out, tokens=tokens, experts=experts)
