"""Pins for the fp64 CPU oracle: worked values, closed forms, invariants, library routines and
brute force on tiny inputs.  None of these re-derives a value through the oracle itself."""
from fractions import Fraction
import os

import numpy as np
import pytest
import scipy.linalg

from oracle import exl3_oracle as O
from moe_exl3_pre_amd import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]


# ------------------------------------------------------------------------------------------ codebook

def test_codebook_worked_values():
    for s, bits, val in _rows("codebook_values.txt"):
        v = O.codebook_value(np.array([int(s, 16)]))[0]
        assert v == float(val), (s, v, val)
        assert np.float16(v).view(np.uint16) == int(bits, 16)


def test_codebook_distribution_closed_form():
    # 0x9E37 is odd, so s -> s*0x9E37 mod 2^16 is a bijection and the 6 masked bits are uniform:
    # 64 values +-2^e (1 + m/8), e in -3..0, m in 0..7, each taken by exactly 1024 states.
    v = O.codebook_value(np.arange(1 << 16))
    expect = sorted(s * 2.0 ** e * (1 + m / 8) for s in (-1, 1) for e in range(-3, 1) for m in range(8))
    vals, counts = np.unique(v, return_counts=True)
    assert list(vals) == expect
    assert np.all(counts == 1024)
    assert v.sum() == 0.0
    # E[v^2] = (1/4 sum_e 4^e) (1/8 sum_m (1+m/8)^2) = (85/256) (1100/512)
    assert np.mean(v * v) == (85 / 256) * (1100 / 512)
    # exact as int8 * 2^-6
    assert np.all(np.abs(v * 64) <= 120) and np.all(v * 64 == np.rint(v * 64))


# ------------------------------------------------------------------------------------------ stream

def _bigint_states(words16, K):
    """Independent reader: the tile's words as one little-endian big integer, doubled for the wrap."""
    n = 256 * K
    stream = 0
    for j, w in enumerate(words16):
        stream |= (int(w) & 0xFFFF) << (16 * j)
    ring = stream | (stream << n)
    return [(ring >> (i * K)) & 0xFFFF for i in range(256)]


def _bit_definition_states(words16, K):
    """The definition as stated: bit j of the stream is bit (j mod 16) of word j // 16."""
    w = np.asarray(words16).astype(np.int64) & 0xFFFF
    n = 256 * K
    bits = [(int(w[j >> 4]) >> (j & 15)) & 1 for j in range(n)]
    return [sum(bits[(i * K + t) % n] << t for t in range(16)) for i in range(256)]


def test_impulse_tail_biting():
    table = {}
    for K, i, s in _rows("impulse_states.txt"):
        table.setdefault(int(K), {})[int(i)] = int(s, 16)
    for K, nz in table.items():
        words = np.zeros(16 * K, dtype=np.int16)
        words[0] = 1
        st = O.tile_states(words, K)
        expect = np.zeros(256, dtype=np.int64)
        for i, s in nz.items():
            expect[i] = s
        assert np.array_equal(st.astype(np.int64), expect), K


def test_all_ones_words():
    for K in range(1, 9):
        words = np.full(16 * K, -1, dtype=np.int16)
        assert np.all(O.tile_states(words, K) == 0xFFFF)
        assert np.all(O.codebook_value(O.tile_states(words, K)) == 0.171875)


@pytest.mark.parametrize("K", range(1, 9))
def test_states_vs_independent_readers(K):
    rng = np.random.default_rng(100 + K)
    tiles = rng.integers(0, 1 << 16, size=(3, 16 * K), dtype=np.uint16).view(np.int16)
    st = O.tile_states(tiles, K)
    for t in range(3):
        assert list(st[t]) == _bigint_states(tiles[t], K)
    assert list(st[0]) == _bit_definition_states(tiles[0], K)


def test_pattern_tile_k3():
    vals = {k: float(v) for k, v in _rows("pattern_tile_k3.txt")}
    words = ((0x1111 * (np.arange(48) + 1)) & 0xFFFF).astype(np.uint16).view(np.int16)
    W = O.decode_weight(words.reshape(1, 1, 48), 3)
    assert W[0, 0] == vals["W00"] and W[15, 0] == vals["W15_0"]
    assert W[0, 1] == vals["W0_1"] and W[15, 15] == vals["W15_15"]
    assert W.sum() == vals["sum"] and (W * W).sum() == vals["sumsq"]


def test_placement_brute_force():
    """W[16a + r, 16b + c] = D(state r + 16c of tile (a, b)), states from the big-int reader and
    values from the fp16 bit pattern read with numpy's own half type."""
    rng = np.random.default_rng(7)
    for K in (2, 3, 5):
        code = synth.random_code(rng, 32, 48, K)
        W = O.decode_weight(code, K)
        for a in range(2):
            for b in range(3):
                st = _bigint_states(code[a, b], K)
                for i in range(256):
                    r, c = i % 16, i // 16
                    p = ((st[i] * 0x9E37) & 0xFFFF) & 0x8F80 | 0x3000
                    v = float(np.array([p], dtype=np.uint16).view(np.float16)[0])
                    assert W[16 * a + r, 16 * b + c] == v


# ------------------------------------------------------------------------------------------ Hadamard

def test_had128_matrix_properties():
    H = O.had128_matrix()
    assert np.max(np.abs(H @ H - np.eye(128))) <= 1e-15
    assert np.array_equal(H, H.T)
    assert np.allclose(H, scipy.linalg.hadamard(128) / np.sqrt(128), atol=0, rtol=0)
    e0 = np.zeros(128); e0[0] = 1
    assert np.allclose(O.had128(e0), np.full(128, 1 / np.sqrt(128)), rtol=1e-15, atol=0)
    assert np.allclose(O.had128(np.ones(128)), np.sqrt(128) * e0, rtol=0, atol=1e-13)


def _fwht(v):
    """In-place radix-2 fast Walsh-Hadamard transform (natural / Sylvester order), normalised."""
    v = np.array(v, dtype=np.float64)
    h = 1
    while h < len(v):
        for i in range(0, len(v), 2 * h):
            a, b = v[i:i + h].copy(), v[i + h:i + 2 * h].copy()
            v[i:i + h], v[i + h:i + 2 * h] = a + b, a - b
        h *= 2
    return v / np.sqrt(len(v))


def test_had128_blockwise_vs_fwht_and_norm():
    rng = np.random.default_rng(3)
    v = rng.standard_normal((3, 512))
    y = O.had128(v)
    for r in range(3):
        for q in range(4):
            assert np.allclose(y[r, 128 * q:128 * q + 128], _fwht(v[r, 128 * q:128 * q + 128]), rtol=0, atol=1e-13)
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(v, axis=1), rtol=1e-14)
    assert np.allclose(O.had128(y), v, rtol=0, atol=1e-13)
    with pytest.raises(ValueError):
        O.had128(np.ones(100))


# ------------------------------------------------------------------------------------------ linear

def _ones(n):
    return np.ones(n)


@pytest.mark.parametrize("fill,val", [(0, 0.125), (-1, 0.171875)])
def test_linear_constant_code_closed_form(fill, val):
    """Constant states make W = v * ones; the output is v * 128 * sum_q t[m, 128q] in column 128p of
    every block and exactly 0 elsewhere (t = x * s_in * rin), times rout * s_out."""
    rng = np.random.default_rng(11)
    M, IC, OC, K = 3, 384, 256, 2
    code = np.full((IC // 16, OC // 16, 16 * K), fill, dtype=np.int16)
    x = rng.standard_normal((M, IC))
    s_in, rin = rng.choice([-1.0, 1.0], IC), rng.uniform(0.5, 1.5, IC)
    rout, s_out = rng.uniform(0.5, 1.5, OC), rng.choice([-1.0, 1.0], OC)
    y = O.linear(x, code, K, s_in, rin, rout, s_out)
    t = x * s_in * rin
    head = val * 128 * t[:, ::128].sum(axis=1)
    expect = np.zeros((M, OC))
    for p in range(OC // 128):
        expect[:, 128 * p] = head * rout[128 * p] * s_out[128 * p]
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-12)
    assert np.all(y[:, 1:128] == 0.0) or np.max(np.abs(y[:, 1:128])) < 1e-12


def test_linear_basis_probe_recovers_rows():
    """x = Had128(e_k) with unit vectors gives xh = e_k, so Had128 of the output is row k of W."""
    rng = np.random.default_rng(5)
    IC, OC, K = 256, 128, 3
    code = synth.random_code(rng, IC, OC, K)
    ks = [0, 17, 130, 255]
    x = np.stack([O.had128(np.eye(IC)[k]) for k in ks])
    y = O.linear(x, code, K, _ones(IC), _ones(IC), _ones(OC), _ones(OC))
    rows = O.had128(y)
    for j, k in enumerate(ks):
        a, r = divmod(k, 16)
        for b in range(OC // 16):
            st = _bigint_states(code[a, b], K)
            for c in range(16):
                p = ((st[r + 16 * c] * 0x9E37) & 0xFFFF) & 0x8F80 | 0x3000
                v = float(np.array([p], dtype=np.uint16).view(np.float16)[0])
                assert abs(rows[j, 16 * b + c] - v) < 1e-12


def test_linear_tiny_brute_force():
    """IC = OC = 128: explicit loops with the explicit Hadamard matrix and the big-int decoder."""
    rng = np.random.default_rng(9)
    M, IC, OC, K = 2, 128, 128, 4
    case = synth.linear_case(9, M, IC, OC, K)
    H = scipy.linalg.hadamard(128) / np.sqrt(128)
    W = np.zeros((IC, OC))
    for a in range(IC // 16):
        for b in range(OC // 16):
            st = _bigint_states(case["code"][a, b], K)
            for i in range(256):
                p = ((st[i] * 0x9E37) & 0xFFFF) & 0x8F80 | 0x3000
                W[16 * a + i % 16, 16 * b + i // 16] = float(np.array([p], dtype=np.uint16).view(np.float16)[0])
    x = case["x"].astype(np.float64)
    s_in, rin = case["s_in"].astype(np.float64), case["rin"].astype(np.float64)
    rout, s_out = case["rout"].astype(np.float64), case["s_out"].astype(np.float64)
    expect = np.zeros((M, OC))
    for m in range(M):
        t = [x[m, k] * s_in[k] * rin[k] for k in range(IC)]
        xh = [sum(H[a, b] * t[b] for b in range(IC)) for a in range(IC)]
        yv = [sum(xh[k] * W[k, n] for k in range(IC)) for n in range(OC)]
        z = [sum(H[a, b] * yv[b] for b in range(OC)) for a in range(OC)]
        expect[m] = [z[n] * rout[n] * s_out[n] for n in range(OC)]
    y = O.linear(case["x"], case["code"], K, case["s_in"], case["rin"], case["rout"], case["s_out"])
    assert np.allclose(y, expect, rtol=1e-12, atol=1e-10)


def test_linear_invariants():
    c = synth.linear_case(21, 4, 256, 384, 3)
    args = (c["code"], 3, c["s_in"], c["rin"], c["rout"], c["s_out"])
    y = O.linear(c["x"], *args)
    # linearity and exact doubling
    assert np.array_equal(O.linear(2 * c["x"].astype(np.float64), *args), 2 * y)
    # s_in -> -s_in negates exactly
    neg = (c["code"], 3, -c["s_in"].astype(np.float64), c["rin"], c["rout"], c["s_out"])
    assert np.array_equal(O.linear(c["x"], *neg), -y)
    # no bias: zero input gives exactly zero
    assert np.all(O.linear(np.zeros_like(c["x"]), *args) == 0.0)
    # rin (pre-scale) and rout (post-scale) are not interchangeable
    IC = 256
    rin2 = np.resize(c["rout"], IC)
    rout2 = np.resize(c["rin"], 384)
    y2 = O.linear(c["x"], c["code"], 3, c["s_in"], rin2, rout2, c["s_out"])
    assert np.max(np.abs(y2 - y)) > 1e-3 * np.max(np.abs(y))
    # rows are independent
    assert np.allclose(O.linear_rows([1, 3], c["x"], *args), y[[1, 3]], rtol=1e-14, atol=1e-12)


def test_merged_equals_concatenation():
    case = synth.merged_case(31, 3, 256, [(128, 2), (256, 3)], shared_input_vectors=False)
    out = np.full((3, case["ldo"]), np.nan)
    pieces = []
    for s in case["shards"]:
        O.linear_into(out, s["col0"], case["x"], s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"])
        pieces.append(O.linear(case["x"], s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"]))
    assert np.array_equal(out, np.concatenate(pieces, axis=1))
    # a slice write leaves the other columns untouched
    out2 = np.full((3, 600), 7.0)
    s = case["shards"][0]
    O.linear_into(out2, 100, case["x"], s["code"], s["K"], s["s_in"], s["rin"], s["rout"], s["s_out"])
    assert np.all(out2[:, :100] == 7.0) and np.all(out2[:, 228:] == 7.0)


def test_fp16_activation_mode_error():
    c = synth.linear_case(41, 8, 1024, 256, 2)
    args = (c["code"], 2, c["s_in"], c["rin"], c["rout"], c["s_out"])
    y = O.linear(c["x"], *args)
    y16 = O.linear(c["x"], *args, act="f16")
    rel = np.linalg.norm(y16 - y) / np.linalg.norm(y)
    assert 1e-5 < rel < 2 ** -11


# ------------------------------------------------------------------------------------------ 8-bit path

def test_int8_quantisation_properties():
    rng = np.random.default_rng(13)
    xh = rng.standard_normal((6, 1024)) * np.array([1, 10, 0.01, 3, 1, 1])[:, None]
    xh[4] = 0.0
    q, sc = O.quantize_rows_int8(xh)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127)
    assert sc[4] == 0 and np.all(q[4] == 0)
    for r in (0, 1, 2, 3, 5):
        assert np.max(np.abs(q[r].astype(int))) == 127
        assert np.max(np.abs(q[r] * sc[r] - xh[r])) <= sc[r] / 2 * (1 + 1e-12)
    q2, sc2 = O.quantize_rows_int8(2 * xh)
    assert np.array_equal(q2, q) and np.array_equal(sc2, 2 * sc)


def test_int8_linear_scale_invariance_and_error():
    c = synth.linear_case(51, 8, 5120 // 4, 256, 3)
    args = (c["code"], 3, c["s_in"], c["rin"], c["rout"], c["s_out"])
    y = O.linear(c["x"], *args)
    y8 = O.linear(c["x"], *args, act="int8")
    assert np.array_equal(O.linear(2 * c["x"].astype(np.float64), *args, act="int8"), 2 * y8)
    rel = np.linalg.norm(y8 - y) / np.linalg.norm(y)
    assert 1e-3 < rel < 3e-2
    zero = O.linear(np.zeros_like(c["x"]), *args, act="int8")
    assert np.all(zero == 0.0)


# ------------------------------------------------------------------------------------------ MoE

def _small_moe(seed=61, T=12, E=6, topk=2, H=256, I=256):
    return synth.moe_case(seed, T=T, E=E, topk=topk, H=H, I=I)


def test_moe_top1_reduces_to_linears():
    m = _small_moe()
    e = m["experts"][3]
    T = m["T"]
    ids = np.full((T, 1), 3, dtype=np.int32)
    w = np.ones((T, 1), dtype=np.float32)
    out = O.moe_forward(m["x"], ids, w, m["experts"])
    one = np.ones(m["H"])
    h1 = O.linear(m["x"], e["w1"], e["k_gu"], e["w1_suh"], 1.0, 1.0, e["w1_svh"])
    h3 = O.linear(m["x"], e["w3"], e["k_gu"], e["w3_suh"], 1.0, 1.0, e["w3_svh"])
    a = h1 / (1 + np.exp(-h1)) * h3
    y = O.linear(a, e["w2"], e["k_d"], e["w2_suh"], one[:m["I"]], 1.0, e["w2_svh"])
    assert np.allclose(out, y, rtol=1e-13, atol=1e-9)


def test_moe_weighted_sum_and_relabel_invariance():
    m = _small_moe()
    out = O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], m["experts"])
    # explicit weighted sum, token by token
    for t in (0, 5):
        acc = np.zeros(m["H"])
        for j in range(m["topk"]):
            acc += float(m["topk_w"][t, j]) * O.expert_forward(m["x"][t:t + 1], m["experts"][m["topk_ids"][t, j]])[0]
        assert np.allclose(out[t], acc, rtol=1e-12, atol=1e-9)
    # relabel experts with a permutation: same output
    perm = np.random.default_rng(1).permutation(m["E"])
    experts2 = [None] * m["E"]
    for e in range(m["E"]):
        experts2[perm[e]] = m["experts"][e]
    out2 = O.moe_forward(m["x"], perm[m["topk_ids"]], m["topk_w"], experts2)
    assert np.allclose(out2, out, rtol=1e-12, atol=1e-9)


def test_moe_unrouted_expert_contributes_nothing():
    m = _small_moe()
    ids = np.where(m["topk_ids"] == 0, 1, m["topk_ids"])
    experts = list(m["experts"])
    experts[0] = dict(experts[0], w1_suh=np.full(m["H"], np.nan))
    out = O.moe_forward(m["x"], ids, m["topk_w"], experts)
    assert np.all(np.isfinite(out))


def test_moe_128_aligned_intermediate_cut_is_exact():
    """Splitting every expert's intermediate dim at a multiple of 128 and summing the two halves
    reproduces the full output (the bank page's rank cut is exact because it is 128-aligned)."""
    m = _small_moe(H=256, I=384)
    cut = 256
    full = O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], m["experts"])
    halves = []
    for lo, hi in ((0, cut), (cut, m["I"])):
        ex = []
        for e in m["experts"]:
            ex.append(dict(e, w1=e["w1"][:, lo // 16:hi // 16], w3=e["w3"][:, lo // 16:hi // 16],
                           w2=e["w2"][lo // 16:hi // 16], w1_svh=e["w1_svh"][lo:hi], w3_svh=e["w3_svh"][lo:hi],
                           w2_suh=e["w2_suh"][lo:hi]))
        halves.append(O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], ex))
    rel = np.linalg.norm(halves[0] + halves[1] - full) / np.linalg.norm(full)
    assert rel <= 1e-12


def test_moe_out_of_range_id_equals_zero_weight():
    """An id outside [0, E) drops its (token, j) term: same result as routing that term to a real expert
    with weight 0 (two different code paths of the dense loop)."""
    m = _small_moe()
    ids = m["topk_ids"].copy()
    w = m["topk_w"].copy()
    ids_bad = ids.copy()
    ids_bad[2, 1] = -1
    ids_bad[7, 0] = m["E"]
    w0 = w.copy()
    w0[2, 1] = 0.0
    w0[7, 0] = 0.0
    a = O.moe_forward(m["x"], ids_bad, w, m["experts"])
    b = O.moe_forward(m["x"], ids, w0, m["experts"])
    assert np.allclose(a, b, rtol=1e-13, atol=1e-9)


def test_moe_token_subset_matches_full():
    m = _small_moe()
    full = O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], m["experts"])
    sub = O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], m["experts"], tokens=[1, 4])
    assert np.allclose(sub[[1, 4]], full[[1, 4]], rtol=1e-12, atol=1e-9)   # BLAS blocking may differ
    assert not np.any(np.delete(sub, [1, 4], axis=0))


def test_moe_f16_operands_close_to_exact():
    """Rounding each projection's rotated input to fp16 perturbs the output by about the fp16 unit
    roundoff (2^-11 relative), far inside the 16-bit path tolerance."""
    m = _small_moe()
    a = O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], m["experts"])
    b = O.moe_forward(m["x"], m["topk_ids"], m["topk_w"], m["experts"], act="f16")
    rel = np.linalg.norm(a - b) / np.linalg.norm(a)
    assert 1e-6 < rel < 2e-3


# ------------------------------------------------------------------------------------------ int8 embedding

def _golden_embed():
    rows = []
    with open(os.path.join(GOLDEN, "embed_int8_values.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                q, s, e = line.split()
                rows.append((int(q), int(s, 16), int(e, 16)))
    return rows


def test_embed_worked_values():
    """Hand-derived products (a tie rounded to even, rounding down and up, exact values, -0)."""
    for q, s, e in _golden_embed():
        table = np.array([[q] * 16], dtype=np.int8)
        got = O.embed_gather(table, np.array([s], dtype=np.uint16), [0])
        assert np.all(got == e), (q, hex(s), hex(int(got[0, 0])), hex(e))


def test_embed_power_of_two_scales_are_exact():
    """With a scale 2^k every int8 code (at most 8 significant bits) is exact in bf16: the result is the
    upper half of the float32 q * 2^k."""
    rng = np.random.default_rng(11)
    table = rng.integers(-128, 128, size=(6, 64), dtype=np.int8)
    ks = np.array([-9, -7, -3, 0, 2, 5])
    sbits = (((ks + 127) << 7)).astype(np.uint16)          # sign 0, exponent k, mantissa 0
    got = O.embed_gather(table, sbits, np.arange(6))
    want = (table.astype(np.float32) * np.ldexp(np.float32(1), ks)[:, None]).astype(np.float32)
    assert np.array_equal(got, (want.view(np.uint32) >> 16).astype(np.uint16))


def test_embed_equals_one_hot_product():
    """The gather is the one-hot row selection of the dequantized table (a matmul with exactly one 1 per
    row adds a single exact term)."""
    rng = np.random.default_rng(12)
    V, H, T = 50, 96, 40
    table = rng.integers(-128, 128, size=(V, H), dtype=np.int8)
    sbits = (rng.integers(0x3B00, 0x3D00, size=V)).astype(np.uint16)
    ids = rng.integers(0, V, size=T)
    onehot = np.zeros((T, V))
    onehot[np.arange(T), ids] = 1.0
    dense = table.astype(np.float64) * O.bf16_bits_to_f64(sbits)[:, None]
    assert np.array_equal(O.embed_gather(table, sbits, ids), O.f64_to_bf16_bits(onehot @ dense))


def test_embed_out_of_range_ids_give_zero_rows():
    rng = np.random.default_rng(13)
    table = rng.integers(-128, 128, size=(8, 32), dtype=np.int8)
    sbits = np.full(8, 0x3F80, dtype=np.uint16)
    got = O.embed_gather(table, sbits, [3, -1, 8, 1 << 20, 3])
    assert np.all(got[1:4] == 0)
    assert np.array_equal(got[0], got[4])
    assert np.array_equal(got[0], (table[3].astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))


def test_bf16_rounding_ties_to_even():
    """Halfway cases of the bf16 rounding go to the even neighbour (both directions)."""
    lo = 1.0 + 2.0 ** -8                                     # halfway between 1 and 1 + 2^-7 -> 1 (even)
    hi = 1.0 + 3 * 2.0 ** -8                                 # halfway between 1 + 2^-7 and 1 + 2^-6 -> 1 + 2^-6
    assert O.f64_to_bf16_bits(np.array([lo]))[0] == 0x3F80
    assert O.f64_to_bf16_bits(np.array([hi]))[0] == 0x3F82
    assert O.f64_to_bf16_bits(np.array([-hi]))[0] == 0xBF82


def test_bf16_rounding_subnormals():
    """Below 2^-126 bf16 numbers lie on the grid 2^-133 (bit patterns 0x0001..0x007F).  Hand values: 1.5,
    2.5 and 3.5 units round to the even neighbour 2, 2, 4; half a unit rounds to zero; a value just below
    2^-126 rounds up to it (0x0080); signs are kept, also for an underflow to zero."""
    u = 2.0 ** -133
    v = np.array([1.5 * u, 2.5 * u, 3.5 * u, 0.5 * u, 0.75 * u, 2.0 ** -126 * (1 - 2.0 ** -10), -1.5 * u, -0.25 * u])
    assert O.f64_to_bf16_bits(v).tolist() == [0x0002, 0x0002, 0x0004, 0x0000, 0x0001, 0x0080, 0x8002, 0x8000]


def test_bf16_rounding_matches_float32_bit_rounding():
    """For float32 inputs (exact in float64) bf16 rounding is the carry trick on the float32 bit pattern,
    (bits + 0x7FFF + bit16) >> 16, which is monotone across the subnormal/normal boundary: every pattern in
    the subnormal range, around 2^-126, and a normal stretch, both signs."""
    pats = np.concatenate([np.arange(0, 1 << 22, 7), np.arange((1 << 23) - 70000, (1 << 23) + 70000),
                           np.arange(0x3F7F0000, 0x3F810000)]).astype(np.uint32)
    pats = np.concatenate([pats, pats | np.uint32(0x80000000)])
    f = pats.view(np.float32)
    want = ((pats.astype(np.uint64) + 0x7FFF + ((pats >> 16) & 1)) >> 16).astype(np.uint16)
    assert np.array_equal(O.f64_to_bf16_bits(f.astype(np.float64)), want)


# ------------------------------------------------------------------------------------------ int8 output head

def _bits(v):
    return O.f64_to_bf16_bits(np.asarray(v, dtype=np.float64))


def test_lm_head_hand_values():
    """Worked by hand.  Rows q = (1, -2) and (3, 4) with scales 0.5 and 0.25 dequantize exactly to (0.5, -1)
    and (0.75, 1); x = (1, 2) gives 0.5 - 2 = -1.5 and 0.75 + 2 = 2.75."""
    got = O.lm_head_int8(_bits([[1.0, 2.0]]), np.array([[1, -2], [3, 4]], dtype=np.int8), _bits([0.5, 0.25]))
    assert np.array_equal(got, _bits([[-1.5, 2.75]]))


def test_lm_head_rounds_each_weight_before_the_sum():
    """The head rounds every dequantized weight to bf16 first.  With s = 1 + 2^-7 the codes 127 and -126
    give 127.9921875 -> 128 and -126.984375 -> -127 (bf16 steps 0.5 in [64, 128)), so x = (1, 1) gives
    exactly 1.0; the unrounded product would be 1.0078125, itself a bf16 number."""
    got = O.lm_head_int8(_bits([[1.0, 1.0]]), np.array([[127, -126]], dtype=np.int8), np.array([0x3F81], np.uint16))
    assert got[0, 0] == 0x3F80


def test_lm_head_identity_rows_give_the_embedding_table():
    """With x the H x H identity each logit is one weight: logits^T equals every row of the table gathered
    and dequantized by the embedding (a separate function of the oracle)."""
    rng = np.random.default_rng(21)
    V, H = 40, 32
    table = rng.integers(-128, 128, size=(V, H), dtype=np.int8)
    sbits = rng.integers(0x3A00, 0x3E00, size=V).astype(np.uint16)
    sbits[::3] |= 0x8000                                  # negative scales too
    got = O.lm_head_int8(_bits(np.eye(H)), table, sbits)
    want = O.embed_gather(table, sbits, np.arange(V))
    # equal up to the sign of a zero: a code 0 under a negative scale gathers as -0 but sums to +0
    assert np.array_equal(O.bf16_bits_to_f64(got.T), O.bf16_bits_to_f64(want))
    assert np.array_equal(got.T & 0x7FFF, want & 0x7FFF)


def _round_bf16_exact(v: Fraction) -> Fraction:
    """Nearest bf16 (8 significant bits, ties to even) of an exact rational, by integer arithmetic."""
    if v == 0:
        return Fraction(0)
    e = 0
    a = abs(v)
    while a >= 256:
        a /= 2
        e += 1
    while a < 128:
        a *= 2
        e -= 1
    n = round(a)                                       # Fraction rounds half to even
    return (1 if v > 0 else -1) * Fraction(n) * Fraction(2) ** e


def test_lm_head_brute_force_exact_rationals():
    """Small random case recomputed with exact rationals and an integer-only bf16 rounding."""
    rng = np.random.default_rng(22)
    M, V, H = 3, 5, 24
    table = rng.integers(-128, 128, size=(V, H), dtype=np.int8)
    sbits = rng.integers(0x3A00, 0x3E00, size=V).astype(np.uint16)
    xbits = _bits(rng.normal(size=(M, H)))
    xf = [[Fraction(float(v)) for v in row] for row in O.bf16_bits_to_f64(xbits)]
    sf = [Fraction(float(v)) for v in O.bf16_bits_to_f64(sbits)]
    got = O.bf16_bits_to_f64(O.lm_head_int8(xbits, table, sbits))
    for m in range(M):
        for v in range(V):
            acc = sum(xf[m][h] * _round_bf16_exact(int(table[v, h]) * sf[v]) for h in range(H))
            assert Fraction(float(got[m, v])) == _round_bf16_exact(acc), (m, v)


def test_lm_head_sign_and_power_of_two_scaling_are_exact():
    rng = np.random.default_rng(23)
    table = rng.integers(-128, 128, size=(16, 64), dtype=np.int8)
    sbits = rng.integers(0x3A00, 0x3E00, size=16).astype(np.uint16)
    x = O.bf16_bits_to_f64(_bits(rng.normal(size=(4, 64))))
    base = O.bf16_bits_to_f64(O.lm_head_int8(_bits(x), table, sbits))
    assert np.array_equal(O.bf16_bits_to_f64(O.lm_head_int8(_bits(-x), table, sbits)), -base)
    assert np.array_equal(O.bf16_bits_to_f64(O.lm_head_int8(_bits(4 * x), table, sbits)), 4 * base)


# ------------------------------------------------------------------------------------------ dense MLP block

def test_silu_identities():
    """silu(g) - silu(-g) = g exactly in real arithmetic, and silu(g) + silu(-g) = g tanh(g/2)."""
    g = np.linspace(-12, 12, 97)
    assert np.allclose(O.silu(g) - O.silu(-g), g, rtol=0, atol=1e-13)
    assert np.allclose(O.silu(g) + O.silu(-g), g * np.tanh(g / 2), rtol=0, atol=1e-13)


def test_silu_mul_hand_values():
    """silu(1) = 1 / (1 + e^-1) = 0.7310585...; 8 significant bits: 1.4621 x 2^-1 -> 187/128 x 2^-1 =
    0.73046875 = 0x3F3B.  silu(64) * 3 rounds to 192 = 0x4340 (silu(64) = 64 (1 - 1.6e-28)).  A zero gate or
    a zero up gives 0."""
    one, three, s64 = 0x3F80, 0x4040, 0x4280
    assert O.silu_mul_bf16(np.array([one]), np.array([one]))[0] == 0x3F3B
    assert O.silu_mul_bf16(np.array([s64]), np.array([three]))[0] == 0x4340
    assert O.bf16_bits_to_f64(O.silu_mul_bf16(np.array([0, one]), np.array([one, 0]))).tolist() == [0.0, 0.0]


def _mlp_case(seed, IC, I, Kg, Ku, Kd):
    rng = np.random.default_rng(seed)

    def proj(ic, oc, K, shared=None):
        p = dict(code=rng.integers(-32768, 32768, size=(ic // 16, oc // 16, 16 * K), dtype=np.int16), K=K,
                 rout=rng.uniform(0.5, 1.5, size=oc), s_out=rng.choice([-1.0, 1.0], size=oc))
        p.update(shared or dict(s_in=rng.choice([-1.0, 1.0], size=ic), rin=rng.uniform(0.5, 1.5, size=ic)))
        return p
    shared = dict(s_in=rng.choice([-1.0, 1.0], size=IC), rin=rng.uniform(0.5, 1.5, size=IC))
    x = O.bf16_bits_to_f64(O.f64_to_bf16_bits(rng.normal(size=(3, IC))))
    return x, proj(IC, I, Kg, shared), proj(IC, I, Ku, shared), proj(I, IC, Kd)


def test_mlp_without_rounding_is_the_expert_forward():
    """With every intermediate kept in float64 and unit rin/rout, the block is the MoE bank's expert MLP
    (a separately pinned function): w1 = gate, w3 = up, w2 = down, suh = s_in, svh = s_out."""
    x, gate, up, down = _mlp_case(31, 256, 384, 2, 2, 3)
    for p in (gate, up, down):
        p["rin"] = np.ones_like(p["rin"])
        p["rout"] = np.ones_like(p["rout"])
    e = dict(w1=gate["code"], w3=up["code"], w2=down["code"], k_gu=2, k_d=3, w1_suh=gate["s_in"],
             w3_suh=up["s_in"], w1_svh=gate["s_out"], w3_svh=up["s_out"], w2_suh=down["s_in"], w2_svh=down["s_out"])
    a = O.mlp_forward(x, gate, up, down, round_mid=False)
    assert np.allclose(a, O.expert_forward(x, e), rtol=1e-12, atol=1e-12)


def test_mlp_rounding_is_small_and_zero_input_gives_zero():
    x, gate, up, down = _mlp_case(32, 256, 384, 2, 3, 3)
    a = O.mlp_forward(x, gate, up, down)
    b = O.mlp_forward(x, gate, up, down, round_mid=False)
    rel = np.linalg.norm(a - b) / np.linalg.norm(b)
    assert 1e-5 < rel < 1e-2
    assert np.all(O.mlp_forward(np.zeros_like(x), gate, up, down) == 0)


# ------------------------------------------------------------------------------------------ rounding points
# Hand-derived values (tests/golden/rounding_points.txt) that fix where the oracle rounds: the fp16
# rounding of the rotated activations comes after the input Hadamard, the 8-bit codes round half to even,
# and the dense MLP block rounds the gate and up outputs to bf16 before its activation.

def _rounding_rows(tag):
    return [r[1:] for r in _rows("rounding_points.txt") if r[0] == tag]


def _zero_code(IC, OC, K=2):
    return np.zeros((IC // 16, OC // 16, 16 * K), dtype=np.int16)


def test_fp16_rounding_point_is_after_the_hadamard():
    rows = _rounding_rows("f16")
    ones = np.ones(128)
    x = np.zeros((len(rows), 128))
    x[:, 0] = [float(c) for c, _, _ in rows]
    got = O.linear(x, _zero_code(128, 128), 2, ones, ones, ones, ones, act="f16")
    for r, (c, num, wrong) in enumerate(rows):
        want = int(num) * np.sqrt(2.0) / 16
        assert abs(got[r, 0] - want) <= 1e-12 * want, (c, got[r, 0], want)
        assert abs(got[r, 0] - float(wrong)) > 1e-3
        assert np.max(np.abs(got[r, 1:])) <= 1e-12 * want
    # the unrounded path gives the "wrong" column: the difference is the fp16 rounding and nothing else
    exact = O.linear(x, _zero_code(128, 128), 2, ones, ones, ones, ones)
    assert np.allclose(exact[:, 0], [float(w) for _, _, w in rows], rtol=1e-12)


def test_int8_codes_round_half_to_even():
    for row in _rounding_rows("i8"):
        sc = float(row[0])
        parts = " ".join(row[1:]).split("|")
        v, even, up, away = ([float(t) for t in p.split()] for p in parts)
        q, s = O.quantize_rows_int8(np.array([v]) * sc)
        assert s[0] == sc
        assert q[0].tolist() == even
        assert q[0].tolist() != up and q[0].tolist() != away


def test_int8_path_takes_the_given_codes():
    """linear(act="int8") is quantize_rows_int8 followed by linear_from_int8; with hand-made codes the
    latter is sc * (q @ W) through the output transform: all-zero words give out[0] = 16 sc q[0]."""
    ones = np.ones(128)
    q = np.zeros((2, 128), dtype=np.int8)
    q[0, 0], q[1, :] = 5, -1
    sc = np.array([0.5, 0.25])
    got = O.linear_from_int8(q, sc, _zero_code(128, 128), 2, ones, ones)
    # out[0] = sqrt(128) * 0.125 * sc * sum_k q[k];  row 1: sum_k q = -128
    want = np.sqrt(128) * 0.125 * sc * np.array([5.0, -128.0])
    assert np.allclose(got[:, 0], want, rtol=1e-13) and np.max(np.abs(got[:, 1:])) < 1e-12
    c = synth.linear_case(52, 5, 256, 128, 3)
    args = (c["code"], 3, c["s_in"], c["rin"], c["rout"], c["s_out"])
    qq, ss = O.quantize_rows_int8(O.rotate_input(c["x"], c["s_in"], c["rin"]))
    assert np.array_equal(O.linear(c["x"], *args, act="int8"),
                          O.linear_from_int8(qq, ss, c["code"], 3, c["rout"], c["s_out"]))


def test_mlp_rounds_gate_and_up_before_the_activation():
    (x0, gbits, ubits, out0, wrong) = _rounding_rows("mlp")[0]
    H = I = 128

    def fp16(bits):
        return float(np.array([int(bits, 16)], dtype=np.uint16).view(np.float16)[0])

    def proj(ic, oc, r0=None):
        rout = np.ones(oc)
        if r0 is not None:
            rout[0] = fp16(r0)
        return dict(code=_zero_code(ic, oc), K=2, s_in=np.ones(ic), rin=np.ones(ic), rout=rout, s_out=np.ones(oc))
    x = np.zeros((1, H))
    x[0, 0] = float(x0)
    gate, up, down = proj(H, I, gbits), proj(H, I, ubits), proj(I, H)
    got = O.mlp_forward(x, gate, up, down)
    assert abs(got[0, 0] - float(out0)) <= 1e-9, got[0, 0]
    assert np.max(np.abs(got[0, 1:])) <= 1e-9
    # with every intermediate in float64 the block gives 16 silu(g) u, not the golden value
    raw = O.mlp_forward(x, gate, up, down, round_mid=False)
    assert abs(raw[0, 0] - float(out0)) > 10 and abs(raw[0, 0] - float(wrong)) < 10
