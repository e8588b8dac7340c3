"""Plain fp64 CPU oracle for the EXL3 trellis-quantized linear layer and its MoE expert bank.

TEST INFRASTRUCTURE ONLY.  Nothing in the product imports this module: only the tests, the
package's smoke check and the CPU-baseline leg of the benchmark call it.  It shares no code,
table or constant generator with the HIP path.

What it computes, and where that comes from
-------------------------------------------
Pages cited (by title):
  [escha]      "radiance_escha.py" -- vLLM quantization method for escha (EXL3 trellis) W2
               checkpoints on gfx1201.  Module docstring: the forward formula
               y = Had128((x*s_in)*rin) @ decode(code) -> Had128 -> *rout -> *s_out, rin is a
               pre-scale, rout a post-scale, bias deliberately not applied.  Constants `_HAD = 128`
               and `_TILE = 16` with the comment "code tensor is [IC//16, OC//16, 16*K]".
               `escha_linear_into`: one projection written into its own column slice.
  [quantpack]  "vllm-quantpack 0.1.0" wheel diff, exl3/linear.py: module docstring ("a packed
               tail-biting trellis ... the bitrate is implied by the trellis width"), and
               `Exl3LinearMethod._forward` (activations cast to fp16 before the GEMM).
  [bank]       "dspark/worker/exl3/bank.py", class `Exl3Bank`: docstring (K-sorted physical slots,
               flat w13 = [w1 | w3] and w2 banks, fp16 suh/svh vectors, 128-aligned intermediate cut).
  [pr190]      "vLLM PR #190: [GG] Add EXL3 Trellis backend for rank-sliced MoE checkpoints":
               commit message describing the dense forward (input suh sign-flip + Hadamard-128,
               trellis GEMM, output svh + Hadamard-128), top-k routing of the MoE plans.

The pages never print the trellis decoder itself (the kernels exist there only as compiled
extensions), so the bit-level reading below is fixed once and used by both sides:

  * tile placement:  code[a, b, :] holds the 16x16 weight tile W[16a:16a+16, 16b:16b+16]
    (W is [IC, OC], y = x @ W).  [escha] `_TILE`; dim0 runs over the input axis, dim1 over the
    output axis.
  * stream:  the tile's 16*K int16 words form a 256*K-bit stream; stream bit j is bit (j mod 16)
    of word floor(j/16).  Equivalently bit (j mod 32) of the j//32-th little-endian uint32 word,
    which is the uint32 reinterpretation [escha] `process_weights_after_loading` hands its kernels.
  * state:  s_i = the 16 stream bits starting at bit i*K, read circularly (tail-biting), least
    significant first:  s_i = sum_t bit((i*K + t) mod 256K) * 2^t,  i in [0, 256).
  * position:  state i lands at tile row r = i mod 16 (input index) and tile column
    c = i div 16 (output index).
  * value:  D(s) = the fp16 number whose bit pattern is ((s * 0x9E37) mod 2^16) & 0x8F80 | 0x3000.
    This is a synthetic codebook (64 distinct values +-2^e (1 + m/8), e in -3..0, m in 0..7);
    the real EXL3 codebooks are not on the pages, so parity with real checkpoints is unpinned.
  * Had128:  the Sylvester-ordered Walsh-Hadamard matrix H[a][b] = (-1)^popcount(a & b) / sqrt(128),
    applied to each consecutive block of 128 features.  It is symmetric and orthogonal.
  * 8-bit activation path:  per row amax = max |xh|, sc = amax / 127, q = clamp(rne(xh / sc), -127, 127)
    ([escha] `escha_linear_into` allocates a uint8 [M, IC] buffer and a float32 [M] scale);
    a row with amax == 0 yields zeros.

Everything here is float64 except where the path itself fixes a narrower type (the fp16 storage
of the decoded weights and scale vectors, and the optional fp16 rounding of the rotated
activations that [quantpack] `_forward` applies).
"""
from __future__ import annotations

import numpy as np

HAD = 128      # [escha] `_HAD`
TILE = 16      # [escha] `_TILE`
STATES = 256   # states per 16x16 tile


# ---------------------------------------------------------------------------------------------
# Trellis decode
# ---------------------------------------------------------------------------------------------

def codebook_value(states: np.ndarray) -> np.ndarray:
    """State -> weight value (the synthetic codebook fixed in the module header), as float64.

    The pages print no codebook; this one is exact in fp16, bf16, fp8-e4m3 and as int8 * 2^-6.
    """
    s = np.asarray(states).astype(np.uint32) & 0xFFFF
    bits = (((s * 0x9E37) & 0xFFFF) & 0x8F80) | 0x3000
    return bits.astype(np.uint16).view(np.float16).astype(np.float64)


def tile_states(tiles: np.ndarray, K: int) -> np.ndarray:
    """The 256 states of each tile: [..., 16K] int16 words -> [..., 256] uint32 states.

    [quantpack] exl3/linear.py docstring: a packed tail-biting trellis whose bitrate K is implied by
    the trellis width ([escha] `_TILE` comment: last dim is 16*K).  State i is the 16-bit window at
    stream bit i*K, read circularly.  The window is taken from the little-endian uint32 view of the
    words: bits [o, o+16) of the stream are bits [o mod 32, o mod 32 + 16) of the 64-bit value
    formed by uint32 word o//32 (low half) and the next word (high half), wrapping to word 0.
    """
    tiles = np.asarray(tiles)
    if tiles.shape[-1] != 16 * K:
        raise ValueError(f"tile width {tiles.shape[-1]} != 16*K = {16 * K}")
    lead = tiles.shape[:-1]
    u16 = np.ascontiguousarray(tiles.reshape(-1, 16 * K)).astype(np.int16).view(np.uint16).astype(np.uint64)
    # little-endian uint32 words: word w = u16[2w] | u16[2w+1] << 16
    u32 = u16[:, 0::2] | (u16[:, 1::2] << np.uint64(16))              # [T, 8K]
    nwords = 8 * K
    offs = np.arange(STATES, dtype=np.int64) * K                       # bit offset of state i
    w0 = offs // 32
    w1 = (w0 + 1) % nwords                                             # tail-biting wrap
    sh = (offs % 32).astype(np.uint64)
    pair = u32[:, w0] | (u32[:, w1] << np.uint64(32))                  # [T, 256] 64-bit windows
    states = (pair >> sh) & np.uint64(0xFFFF)
    return states.astype(np.uint32).reshape(*lead, STATES)


def decode_weight(code: np.ndarray, K: int) -> np.ndarray:
    """Dense weight W [IC, OC] (float64) of a code tensor int16 [IC/16, OC/16, 16K].

    [escha] `_TILE`: code[a, b] holds W[16a:16a+16, 16b:16b+16]; state i sits at in-tile row
    i mod 16 (input index) and column i div 16 (output index).
    """
    code = np.asarray(code)
    if code.ndim != 3 or code.shape[2] != 16 * K:
        raise ValueError(f"code shape {code.shape} is not [IC/16, OC/16, 16*{K}]")
    A, B = code.shape[0], code.shape[1]
    W = np.empty((A, TILE, B, TILE), dtype=np.float64)
    chunk = max(1, 65536 // max(B, 1))
    for a0 in range(0, A, chunk):
        a1 = min(A, a0 + chunk)
        v = codebook_value(tile_states(code[a0:a1], K))                # [a, B, 256]
        v = v.reshape(a1 - a0, B, TILE, TILE)                          # [a, B, c, r] (i = 16c + r)
        W[a0:a1] = v.transpose(0, 3, 1, 2)                             # [a, r, B, c]
    return W.reshape(A * TILE, B * TILE)


# ---------------------------------------------------------------------------------------------
# Hadamard-128
# ---------------------------------------------------------------------------------------------

def had128_matrix() -> np.ndarray:
    """Orthonormal Sylvester Hadamard matrix of order 128 ([escha] `_HAD`; [pr190] Hadamard-128)."""
    H = np.ones((1, 1), dtype=np.float64)
    while H.shape[0] < HAD:
        H = np.block([[H, H], [H, -H]])
    return H / np.sqrt(HAD)


def had128(v: np.ndarray, axis: int = -1) -> np.ndarray:
    """Apply Had128 to every consecutive 128-block along `axis` ([escha]: the transform is blocked at 128)."""
    v = np.asarray(v, dtype=np.float64)
    v = np.moveaxis(v, axis, -1)
    n = v.shape[-1]
    if n % HAD:
        raise ValueError(f"length {n} is not a multiple of {HAD}")
    blocks = v.reshape(*v.shape[:-1], n // HAD, HAD)
    out = blocks @ had128_matrix()          # H is symmetric, so row-vector times H == H times column
    return np.moveaxis(out.reshape(v.shape), -1, axis)


# ---------------------------------------------------------------------------------------------
# The linear layer
# ---------------------------------------------------------------------------------------------

def round_fp16(v: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest fp16 (ties to even), returned as float64."""
    return np.asarray(v, dtype=np.float64).astype(np.float16).astype(np.float64)


def rotate_input(x, s_in, rin) -> np.ndarray:
    """xh = Had128((x * s_in) * rin) along the input features ([escha] module docstring: rin is a
    pre-scale applied before its Hadamard; [pr190]: input sign flip + Hadamard-128)."""
    x = np.asarray(x, dtype=np.float64)
    t = x * np.asarray(s_in, dtype=np.float64) * np.asarray(rin, dtype=np.float64)
    return had128(t, axis=-1)


def quantize_rows_int8(xh: np.ndarray):
    """Per-row symmetric 8-bit quantisation of the rotated activations.

    [escha] `escha_linear_into` stages an 8-bit [M, IC] buffer, a float32 [M] scale and a
    zero-initialised [M] amax.  Reading: sc = amax/127, q = clamp(round-half-even(xh/sc), -127, 127);
    a row with amax == 0 gets sc = 0 and q = 0.  Returns (q int8 [M, IC], sc float64 [M]).
    """
    xh = np.asarray(xh, dtype=np.float64)
    amax = np.max(np.abs(xh), axis=-1) if xh.shape[-1] else np.zeros(xh.shape[:-1])
    sc = amax / 127.0
    safe = np.where(sc > 0, sc, 1.0)
    q = np.clip(np.rint(xh / safe[..., None]), -127, 127)
    q = np.where(sc[..., None] > 0, q, 0.0)
    return q.astype(np.int8), sc


def linear(x, code, K, s_in, rin, rout, s_out, act: str = "f64", W: np.ndarray | None = None) -> np.ndarray:
    """One EXL3 projection, float64, before the output's bf16 rounding.

    [escha] module docstring:  y = Had128((x*s_in)*rin) @ decode(code) -> Had128 -> *rout -> *s_out,
    with no bias.  x is [M, IC]; returns [M, OC].

    act selects how the rotated activations enter the product:
      "f64"  -- exact;
      "f16"  -- rounded once to fp16, as [quantpack] `_forward` casts before its GEMM;
      "int8" -- the per-row 8-bit path of `quantize_rows_int8`, product rescaled by the row scale.
    """
    if W is None:
        W = decode_weight(code, K)
    xh = rotate_input(x, s_in, rin)
    if act == "f64":
        Y = xh @ W
    elif act == "f16":
        Y = round_fp16(xh) @ W
    elif act == "int8":
        q, sc = quantize_rows_int8(xh)
        return linear_from_int8(q, sc, code, K, rout, s_out, W=W)
    else:
        raise ValueError(f"unknown act mode {act!r}")
    return output_transform(Y, rout, s_out)


def output_transform(Y, rout, s_out) -> np.ndarray:
    """Z = Had128(Y) along the output features, then * rout * s_out ([escha] module docstring: the
    product is followed by its own Hadamard-128 and the post-scales; no bias)."""
    Z = had128(Y, axis=-1)
    return Z * np.asarray(rout, dtype=np.float64) * np.asarray(s_out, dtype=np.float64)


def linear_from_int8(q, sc, code, K, rout, s_out, W: np.ndarray | None = None) -> np.ndarray:
    """The 8-bit path after its quantisation step: Y = sc[m] * (q @ W), then the output transform.

    q is [M, IC] (integers in [-127, 127]) and sc the [M] row scales, as `quantize_rows_int8` returns them
    ([escha] `escha_linear_into`: the 8-bit activation buffer and its float32 row scale feed the GEMM).
    Taking q and sc as arguments lets a test run this step on codes another implementation chose."""
    if W is None:
        W = decode_weight(code, K)
    q = np.asarray(q).astype(np.float64)
    sc = np.asarray(sc, dtype=np.float64)
    return output_transform(sc[:, None] * (q @ W), rout, s_out)


def linear_into(out: np.ndarray, col0: int, x, code, K, s_in, rin, rout, s_out, act: str = "f64") -> np.ndarray:
    """[escha] `escha_linear_into`: write one projection into columns [col0, col0 + OC) of `out`
    (float64 [M, ldo]); every other column is left untouched."""
    y = linear(x, code, K, s_in, rin, rout, s_out, act=act)
    out[:, col0:col0 + y.shape[1]] = y
    return out


def linear_rows(rows, x, code, K, s_in, rin, rout, s_out, act: str = "f64", W=None) -> np.ndarray:
    """The same projection evaluated for a subset of rows only (rows are independent)."""
    x = np.asarray(x)[np.asarray(rows)]
    return linear(x, code, K, s_in, rin, rout, s_out, act=act, W=W)


# ---------------------------------------------------------------------------------------------
# MoE expert bank
# ---------------------------------------------------------------------------------------------

def silu(h: np.ndarray) -> np.ndarray:
    """SiLU(h) = h / (1 + exp(-h))."""
    h = np.asarray(h, dtype=np.float64)
    return h / (1.0 + np.exp(-h))


def expert_forward(v, e, act: str = "f64") -> np.ndarray:
    """One expert's MLP on rows v [n, H]: w2( silu(w1 v) * (w3 v) ), each an EXL3 projection whose
    input sign/scale vector is its suh and whose output vector is its svh ([bank] docstring: w13_suh,
    w13_svh, w2_suh, w2_svh; [pr190]: input suh + Hadamard-128, output svh + Hadamard-128).

    `e` is a dict with keys w1, w3 (int16 [H/16, I/16, 16 k_gu]), w2 (int16 [I/16, H/16, 16 k_d]),
    k_gu, k_d, w1_suh, w3_suh [H], w1_svh, w3_svh [I], w2_suh [I], w2_svh [H].  Optional pre-decoded
    dense weights may be given as W1, W3, W2.  `act` is passed to each of the three projections
    ("f16": every projection's rotated input is rounded once to fp16; h1, h3 and the silu product are
    not rounded).
    """
    ones_h = 1.0
    h1 = linear(v, e["w1"], e["k_gu"], e["w1_suh"], ones_h, ones_h, e["w1_svh"], act=act, W=e.get("W1"))
    h3 = linear(v, e["w3"], e["k_gu"], e["w3_suh"], ones_h, ones_h, e["w3_svh"], act=act, W=e.get("W3"))
    a = silu(h1) * h3
    return linear(a, e["w2"], e["k_d"], e["w2_suh"], ones_h, ones_h, e["w2_svh"], act=act, W=e.get("W2"))


def moe_forward(x, topk_ids, topk_w, experts, act: str = "f64", tokens=None) -> np.ndarray:
    """Dense per-expert loop over logical expert ids:
       out[t] = sum_j topk_w[t, j] * E_{topk_ids[t, j]}(x[t])            (float64 [T, H]).

    `experts[e]` is the dict of `expert_forward` for logical expert e.  Experts that receive no
    token are never evaluated and contribute nothing; ids outside [0, E) contribute nothing.  With
    `tokens` given, only those rows are computed (the others stay zero).
    """
    x = np.asarray(x, dtype=np.float64)
    ids = np.asarray(topk_ids)
    w = np.asarray(topk_w, dtype=np.float64)
    T = x.shape[0]
    out = np.zeros_like(x)
    keep = np.zeros(T, dtype=bool)
    keep[np.arange(T) if tokens is None else np.asarray(tokens)] = True
    for ex in np.unique(ids):
        if ex < 0 or ex >= len(experts):
            continue
        tok, slot = np.nonzero((ids == ex) & keep[:, None])
        if tok.size == 0:
            continue
        y = expert_forward(x[tok], experts[int(ex)], act=act)
        np.add.at(out, tok, w[tok, slot][:, None] * y)
    assert out.shape[0] == T
    return out


# ---------------------------------------------------------------------------------------------
# int8 embedding rows gathered and dequantized
# ---------------------------------------------------------------------------------------------
# [quantpack] exl3/embedding.py, `Exl3EmbeddingMethod.embedding`: the table stays int8 with one scale per
# row; the rows of the requested token ids are gathered, converted to the scale's dtype (bf16 here) and
# multiplied by their row's scale.  An int8 code times a bf16 scale is exact in any binary format with
# 16 or more significand bits, so the result is that exact product rounded once to bf16 (nearest, ties
# to even).  Ids outside [0, V) give zero rows: the reading of the page's tensor-parallel cut, where
# VocabParallelEmbedding masks the ids a rank does not hold.

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) to float64: a bf16 number is the upper half of a float32."""
    b = np.asarray(bits, dtype=np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even) and return the bit patterns.  bf16 keeps 8
    significant bits down to 2^-126; below that its numbers (subnormals) lie on the fixed grid 2^-133, so
    the rounding unit is 2^(e-8) for v = m 2^e, 1/2 <= |m| < 1, but never below 2^-133.  Values past the
    largest bf16 are not handled (none arises here); zeros keep their sign."""
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    unit = np.maximum(e - 8, -133)                       # exponent of the rounding unit
    r = np.ldexp(np.rint(np.ldexp(v, -unit)), unit)      # np.rint rounds half to even
    r = np.where(r == 0, np.copysign(0.0, v), r)         # keep the sign of zero (also of an underflow)
    return (r.astype(np.float32).view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def embed_gather(table_q: np.ndarray, scale_bits: np.ndarray, ids) -> np.ndarray:
    """out[t, :] = bf16(table_q[ids[t], :] * scale[ids[t]]) as bf16 bit patterns [T, H] (uint16);
    zero rows for ids outside [0, V)."""
    table_q = np.asarray(table_q, dtype=np.int8)
    V, H = table_q.shape
    ids = np.asarray(ids, dtype=np.int64).reshape(-1)
    s = bf16_bits_to_f64(np.asarray(scale_bits, dtype=np.uint16).reshape(-1))
    rows = np.zeros((ids.size, H), dtype=np.float64)
    ok = (ids >= 0) & (ids < V)
    rows[ok] = table_q[ids[ok]].astype(np.float64) * s[ids[ok]][:, None]
    return f64_to_bf16_bits(rows)


# ---------------------------------------------------------------------------------------------
# int8 table used as the output head (tied embedding / lm_head)
# ---------------------------------------------------------------------------------------------
# [quantpack] exl3/embedding.py, `Exl3EmbeddingMethod.apply`: the head multiplies the whole int8 table
# by its row scales in the activations' dtype (bf16), so every weight is rounded once, w[v, h] =
# bf16(q[v, h] * s[v]); the logits are the linear map x @ w^T, rounded once to bf16.  Here the sum is
# taken in float64 before that rounding.  No bias: a tied head has none (the page adds one only when
# given).

def lm_head_int8(x_bits: np.ndarray, table_q: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """logits[m, v] = bf16(sum_h x[m, h] * bf16(q[v, h] * s[v])) as bf16 bit patterns [M, V] (uint16).
    x_bits: [M, H] bf16 bit patterns; table_q: [V, H] int8; scale_bits: [V] bf16 bit patterns."""
    x = bf16_bits_to_f64(np.asarray(x_bits, dtype=np.uint16))
    q = np.asarray(table_q, dtype=np.int8).astype(np.float64)
    s = bf16_bits_to_f64(np.asarray(scale_bits, dtype=np.uint16).reshape(-1))
    w = bf16_bits_to_f64(f64_to_bf16_bits(q * s[:, None]))
    return f64_to_bf16_bits(x @ w.T)


# ---------------------------------------------------------------------------------------------
# Dense MLP block: merged gate/up, SiLU * mul, down
# ---------------------------------------------------------------------------------------------
# [quantpack] exl3/linear.py module docstring: gate and up are two shards of one fused gate_up layer (their
# own EXL3 tensors, possibly of different K) whose outputs are concatenated; the model's activation then
# takes silu(gate) * up and feeds down_proj.  Reading: the serving stack's dense block, where the fused
# layer's output is bf16, the activation is evaluated on those bf16 values and rounded once to bf16, and
# down_proj consumes that bf16 tensor.  (The MoE bank above keeps its intermediates in fp32 instead.)

def silu_mul_bf16(g_bits: np.ndarray, u_bits: np.ndarray) -> np.ndarray:
    """h = bf16(silu(g) * u) for bf16 bit patterns g, u of the same shape; returns bf16 bit patterns."""
    g = bf16_bits_to_f64(np.asarray(g_bits, dtype=np.uint16))
    u = bf16_bits_to_f64(np.asarray(u_bits, dtype=np.uint16))
    return f64_to_bf16_bits(silu(g) * u)


def mlp_forward(x, gate: dict, up: dict, down: dict, act: str = "f64", round_mid: bool = True) -> np.ndarray:
    """down( silu(gate(x)) * up(x) ), float64 before the output's bf16 rounding.

    gate, up and down are dicts with keys code, K, s_in, rin, rout, s_out (the arguments of `linear`).  With
    round_mid the gate and up outputs are rounded to bf16 and the activation is rounded to bf16 (the reading
    above); without it every intermediate stays float64.  `act` is passed to each projection."""
    def proj(v, p):
        return linear(v, p["code"], p["K"], p["s_in"], p["rin"], p["rout"], p["s_out"], act=act)
    g, u = proj(x, gate), proj(x, up)
    if round_mid:
        h = bf16_bits_to_f64(silu_mul_bf16(f64_to_bf16_bits(g), f64_to_bf16_bits(u)))
    else:
        h = silu(g) * u
    return proj(h, down)
