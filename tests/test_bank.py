"""Host-side MoE bank packing and the MoE entry point's argument checks (no GPU needed)."""
import ctypes

import numpy as np
import pytest

from moe_exl3_pre_amd import exl3, synth
from moe_exl3_pre_amd.bank import pack_bank

FAKE = 0x10000


def _case(**kw):
    a = dict(seed=3, T=8, E=9, topk=2, H=256, I=128, Ks=(2, 3, 4))
    a.update(kw)
    return synth.moe_case(a.pop("seed"), **a)


def test_projection_views_round_trip_every_slot():
    m = _case(k_d_independent=True)
    b = pack_bank(m["experts"], m["H"], m["I"])
    for e, ex in enumerate(m["experts"]):
        (w1, s1, v1, k1), (w3, s3, v3, k3), (w2, s2, v2, k2) = (b.projection(int(b.perm[e]), n)
                                                                 for n in ("w1", "w3", "w2"))
        assert k1 == k3 == ex["k_gu"] and k2 == ex["k_d"]
        assert np.array_equal(w1, ex["w1"]) and np.array_equal(w3, ex["w3"]) and np.array_equal(w2, ex["w2"])
        assert np.array_equal(s1, ex["w1_suh"]) and np.array_equal(s3, ex["w3_suh"]) and np.array_equal(s2, ex["w2_suh"])
        assert np.array_equal(v1, ex["w1_svh"]) and np.array_equal(v3, ex["w3_svh"]) and np.array_equal(v2, ex["w2_svh"])


def test_slots_sorted_stably_and_groups_are_maximal_runs():
    m = _case(E=12, k_d_independent=True)
    b = pack_bank(m["experts"], m["H"], m["I"])
    keys = [(e["k_gu"], e["k_d"]) for e in m["experts"]]
    order = np.argsort(b.perm)                      # slot -> logical
    assert sorted(b.perm.tolist()) == list(range(12))
    slot_keys = [keys[e] for e in order]
    assert slot_keys == sorted(slot_keys)
    for p in range(11):                             # stable: equal keys keep logical order
        if slot_keys[p] == slot_keys[p + 1]:
            assert order[p] < order[p + 1]
    lo = 0
    for kg, kd, glo, ghi in b.groups:
        assert glo == lo and ghi > glo
        assert all(slot_keys[p] == (kg, kd) for p in range(glo, ghi))
        lo = ghi
    assert lo == 12
    for (_, _, _, h1), (_, _, l2, _) in zip(b.groups, b.groups[1:]):
        assert slot_keys[h1 - 1] != slot_keys[l2]


def test_offsets_are_prefix_sums_and_aligned():
    m = _case(E=7)
    b = pack_bank(m["experts"], m["H"], m["I"])
    n13 = m["H"] * m["I"] * b.k_gu // 16
    n2 = m["H"] * m["I"] * b.k_d // 16
    assert np.array_equal(b.off_w3, b.off_w1 + n13)
    assert np.array_equal(b.off_w1[1:], b.off_w1[:-1] + 2 * n13[:-1])
    assert np.array_equal(b.off_w2[1:], b.off_w2[:-1] + n2[:-1])
    assert b.w13.size == b.off_w1[-1] + 2 * n13[-1] and b.w2.size == b.off_w2[-1] + n2[-1]
    assert np.all(b.off_w1 % 8 == 0) and np.all(b.off_w3 % 8 == 0) and np.all(b.off_w2 % 8 == 0)   # 16-byte
    assert b.trellis_bytes() == 2 * (b.w13.size + b.w2.size)


def test_pack_rejects_wrong_shape():
    m = _case()
    m["experts"][2] = dict(m["experts"][2], w2=m["experts"][2]["w2"][:, :-1])
    with pytest.raises(ValueError, match="expert 2 w2"):
        pack_bank(m["experts"], m["H"], m["I"])


# ---------------------------------------------------------------------------------------- ABI checks

def _bank(**kw):
    groups = kw.pop("groups", [(2, 2, 0, 4), (3, 3, 4, 8)])
    g = (exl3.Group * max(len(groups), 1))(*[exl3.Group(*x) for x in groups])
    a = dict(E=8, H=256, I=128, n_groups=len(groups), w13=FAKE, w2=FAKE, w13_suh=FAKE, w13_svh=FAKE, w2_suh=FAKE,
             w2_svh=FAKE, off_w1=FAKE, off_w3=FAKE, off_w2=FAKE, perm=FAKE)
    a.update(kw)
    b = exl3.Bank(a["E"], a["H"], a["I"], a["n_groups"], a["w13"], a["w2"], a["w13_suh"], a["w13_svh"], a["w2_suh"],
                  a["w2_svh"], a["off_w1"], a["off_w3"], a["off_w2"], a["perm"], ctypes.cast(g, ctypes.POINTER(exl3.Group)))
    b._keep = g
    return b


def _fwd(bank, T=4, topk=2, flags=0, ws=FAKE, ws_bytes=1 << 30, out=FAKE, x=FAKE, ids=FAKE, w=FAKE):
    return exl3.lib().exl3_moe_bank_forward(out, x, T, ids, w, topk, ctypes.byref(bank), flags, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,fkw,code,needle", [
    (dict(E=0), {}, exl3.EINVAL, "bank.E"),
    (dict(E=2000), {}, exl3.EINVAL, "bank.E"),
    (dict(H=200), {}, exl3.EINVAL, "bank.H"),
    (dict(I=0), {}, exl3.EINVAL, "bank.I"),
    (dict(n_groups=0, groups=[]), {}, exl3.EINVAL, "bank.n_groups"),
    (dict(groups=[(2, 2, 0, 4), (3, 3, 5, 8)]), {}, exl3.EINVAL, "bank.groups[1]"),
    (dict(groups=[(2, 2, 0, 4), (3, 3, 4, 7)]), {}, exl3.EINVAL, "bank.groups"),
    (dict(groups=[(2, 9, 0, 8)]), {}, exl3.EINVAL, "k_d"),
    (dict(w13=None), {}, exl3.EINVAL, "bank.w13"),
    (dict(w2=FAKE + 8), {}, exl3.EINVAL, "bank.w13/w2"),
    (dict(w2_svh=None), {}, exl3.EINVAL, "w2_svh"),
    (dict(w13_suh=FAKE + 2), {}, exl3.EINVAL, "w13_suh"),
    (dict(off_w3=FAKE + 4), {}, exl3.EINVAL, "off_w"),
    (dict(perm=None), {}, exl3.EINVAL, "bank.perm"),
    ({}, dict(topk=0), exl3.EINVAL, "topk"),
    ({}, dict(topk=9), exl3.EINVAL, "topk"),
    ({}, dict(T=-1), exl3.EINVAL, "T"),
    ({}, dict(flags=exl3.ACT_INT8), exl3.EUNSUPPORTED, "flags"),
    ({}, dict(flags=exl3.GEMM_NO_SPLIT), exl3.EINVAL, "flags"),
    ({}, dict(flags=exl3.FORCE_GEMV | exl3.FORCE_MFMA), exl3.EINVAL, "exclusive"),
    ({}, dict(out=None), exl3.EINVAL, "out"),
    ({}, dict(x=FAKE + 2), exl3.EINVAL, "x"),
    ({}, dict(ids=None), exl3.EINVAL, "topk_ids"),
    ({}, dict(w=FAKE + 2), exl3.EINVAL, "topk_w"),
    ({}, dict(ws=None), exl3.EWORKSPACE, "ws"),
    ({}, dict(ws_bytes=4096), exl3.EWORKSPACE, "ws_bytes"),
])
def test_moe_rejects_before_launch(kw, fkw, code, needle):
    rc = _fwd(_bank(**kw), **fkw)
    assert rc == code, (rc, exl3.last_error())
    assert needle in exl3.last_error()


def test_moe_zero_tokens_is_a_noop():
    assert _fwd(_bank(), T=0, out=None, x=None, ids=None, w=None) == exl3.OK


def test_moe_workspace_grows_with_tokens():
    b = _bank()
    sizes = [exl3.lib().exl3_moe_workspace_bytes(ctypes.byref(b), T, 2, 0) for T in (1, 16, 256)]
    assert sizes == sorted(sizes) and all(s % 256 == 0 for s in sizes)
    # per pair: rotated w1/w3 inputs (2 H fp16), w2 operand (I fp16), expert output (H fp32)
    assert sizes[2] - sizes[1] >= 240 * 2 * (2 * 256 * 2 + 128 * 2 + 256 * 4)
