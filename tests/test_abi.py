"""Host-side checks of the C ABI: the library loads, exports every declared symbol, and rejects bad
arguments before launching anything.  No call here reaches a kernel (no GPU needed)."""
import ctypes
import os
import re

import pytest

from moe_exl3_pre_amd import exl3

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "exl3.h")

FAKE = 0x10000           # 64 KiB-aligned fake device address: never dereferenced by host validation


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(exl3_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = exl3.lib()
    declared = _declared_functions()
    assert len(declared) >= 10
    for name in declared:
        assert hasattr(L, name), name
    assert sorted(declared) == sorted(exl3.exported_symbols())


def test_version_and_limits():
    L = exl3.lib()
    assert L.exl3_version() >= 100
    # the measured crossover rule against the (feature-split) GEMM: 16 * clamp(10240 // OC, 2, 8)
    for OC, rows in ((17408, 32), (14336, 32), (7168, 32), (5120, 32), (4096, 32), (2560, 64), (1024, 128),
                     (256, 128), (81920, 32)):
        assert L.exl3_gemv_max_rows(OC) == rows, OC


def _linear(**kw):
    a = dict(out=FAKE, ldo=512, col0=0, x=FAKE, M=4, IC=512, code=FAKE, OC=512, K=3, s_in=FAKE, rin=FAKE, rout=FAKE,
             s_out=FAKE, flags=0, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return exl3.lib().exl3_linear_into(a["out"], a["ldo"], a["col0"], a["x"], a["M"], a["IC"], a["code"], a["OC"],
                                       a["K"], a["s_in"], a["rin"], a["rout"], a["s_out"], a["flags"], a["ws"],
                                       a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code,needle", [
    (dict(IC=500), exl3.EINVAL, "IC"),
    (dict(IC=0), exl3.EINVAL, "IC"),
    (dict(OC=300), exl3.EINVAL, "OC"),
    (dict(K=0), exl3.EINVAL, "K"),
    (dict(K=9), exl3.EINVAL, "K"),
    (dict(col0=100), exl3.EINVAL, "col0"),
    (dict(col0=-1), exl3.EINVAL, "col0"),
    (dict(M=-1), exl3.EINVAL, "M"),
    (dict(code=None), exl3.EINVAL, "code"),
    (dict(code=FAKE + 2), exl3.EINVAL, "code"),
    (dict(s_in=None), exl3.EINVAL, "s_in"),
    (dict(rin=FAKE + 2), exl3.EINVAL, "rin"),
    (dict(rout=None), exl3.EINVAL, "rout"),
    (dict(x=None), exl3.EINVAL, "x"),
    (dict(x=FAKE + 4), exl3.EINVAL, "x"),
    (dict(out=None), exl3.EINVAL, "out"),
    (dict(flags=1 << 7), exl3.EINVAL, "flags"),
    (dict(flags=exl3.ACT_INT8 | exl3.FORCE_GEMV, ws=None), exl3.EWORKSPACE, "ws"),  # 8-bit decode phase accepted
    (dict(flags=exl3.ACT_INT8, ws=None), exl3.EWORKSPACE, "ws"),              # 8-bit path accepted
    (dict(flags=exl3.FORCE_GEMV | exl3.FORCE_MFMA), exl3.EINVAL, "flags"),
    (dict(flags=exl3.BATCH_INVARIANT | exl3.FORCE_MFMA), exl3.EINVAL, "BATCH_INVARIANT"),
    (dict(flags=exl3.BATCH_INVARIANT | exl3.ACT_INT8, ws=None), exl3.EWORKSPACE, "ws"),  # accepted
    (dict(ws=None), exl3.EWORKSPACE, "ws"),
    (dict(ws=FAKE, ws_bytes=1024), exl3.EWORKSPACE, "ws_bytes"),
    (dict(ws=FAKE + 16, ws_bytes=1 << 30), exl3.EINVAL, "ws"),
])
def test_linear_rejects_before_launch(kw, code, needle):
    rc = _linear(**kw)
    assert rc == code, (rc, exl3.last_error())
    assert needle in exl3.last_error()


def test_linear_zero_rows_is_a_noop():
    assert _linear(M=0, out=None, x=None) == exl3.OK
    assert exl3.last_error() == ""


def test_int8_workspace_holds_codes_and_scales():
    """The 8-bit path runs on the GEMM at every M: its workspace holds M x IC fp16 codes plus M scales."""
    for M in (1, 4, 300):
        assert exl3.linear_workspace_bytes(M, 4096, 14336, exl3.ACT_INT8) >= 16384 + M * 4096 * 2 + M * 4


def test_embed_validation():
    """Host-side checks of the embedding gather (no launch): H a positive multiple of 16, V >= 1, T >= 0,
    non-null pointers; T == 0 is a no-op."""
    L = exl3.lib()
    assert L.exl3_embed_int8(None, None, None, 10, 24, None, 4, None) == -1
    assert L.exl3_embed_int8(None, None, None, 0, 32, None, 4, None) == -1
    assert L.exl3_embed_int8(None, None, None, 10, 32, None, -1, None) == -1
    assert L.exl3_embed_int8(None, None, None, 10, 32, None, 3, None) == -1
    assert b"null" in L.exl3_last_error()
    assert L.exl3_embed_int8(None, None, None, 10, 32, None, 0, None) == 0


def test_gemm_tail_split_plan():
    """Large shards whose 4-wave blocks (128 x 512) leave the last round of 256 at most half full split
    that round's blocks over the input features; the workspace holds their partial tiles."""
    L = exl3.lib()
    # (M, IC, OC) -> blocks = ceil(M/128) * ceil(OC/512)
    for M, IC, OC, want in ((8192, 5120, 17408, 2),      # 2176 blocks: 128 in the last round
                            (8192, 17408, 5120, 2),      # 640 blocks: 128 in the last round
                            (1152, 1024, 14848, 2),      # 261 blocks: 5, capped at 2 by 16 steps
                            (8192, 4096, 16384, 1),      # 2048 blocks: whole rounds
                            (8192, 4096, 18432, 1),      # 2304 blocks: 0 left over
                            (8192, 4096, 17920, 1)):     # 2240 blocks: 192 left over, more than half
        assert L.exl3_gemm_splits(M, IC, OC) == 1
        assert L.exl3_gemm_tail_splits(M, IC, OC) == want, (M, IC, OC)
    assert L.exl3_gemm_tail_splits(8192, 1024, 8192 + 512) == 2   # 17 * 64 = 1088 blocks: 64 left over
    assert L.exl3_gemm_tail_splits(200, 2048, 256) == 1           # a fully split shard has no tail split
    ws = exl3.linear_workspace_bytes(8192, 17408, 5120)
    assert ws >= 16384 + 2 * 128 * 4 * 65536 + 8192 * 17408 * 2
    assert exl3.linear_workspace_bytes(8192, 17408, 5120, exl3.GEMM_NO_SPLIT) < ws


def test_int8_decode_workspace_holds_codes_scales_and_maxima():
    """The 8-bit path on the decode-phase kernel writes its codes at every M: 16 (32) rows x IC fp16, plus the
    row scales and the per-(row, 128-block) maxima, per distinct (s_in, rin); the 16-bit path needs no region
    below 5 rows."""
    IC, OC = 2048, 28672
    for M, rows in ((1, 16), (4, 16), (16, 16), (17, 32), (32, 32)):
        f16 = exl3.linear_workspace_bytes(M, IC, OC)
        i8 = exl3.linear_workspace_bytes(M, IC, OC, exl3.ACT_INT8)
        assert i8 >= 16384 + rows * IC * 2 + rows * 4 + rows * (IC // 128) * 4, (M, i8)
        assert i8 > f16, (M, i8, f16)
        assert exl3.linear_workspace_bytes(M, IC, OC, exl3.ACT_INT8 | exl3.FORCE_GEMV) == i8


def test_decode_workspace_pre_rotation_region():
    """Decode-phase launches of 5..32 rows rotate the activations once per call into the workspace
    (fragment-major 16-row blocks: 16 rows x IC fp16 up to 16 rows, 32 above); below 5 rows each block
    rotates its own.  A 28672-column shard over IC=2048 needs no split-K slab, so the workspace is the
    counter area plus that region."""
    IC, OC = 2048, 28672
    assert exl3.lib().exl3_gemv_max_rows(OC) >= 32
    for M in (1, 4):
        assert exl3.linear_workspace_bytes(M, IC, OC) == 16384
    for M in (5, 8, 16):
        assert exl3.linear_workspace_bytes(M, IC, OC) == 16384 + 16 * IC * 2
    for M in (17, 32):
        assert exl3.linear_workspace_bytes(M, IC, OC) == 16384 + 32 * IC * 2


def test_workspace_sizes():
    """256-byte multiples, never below the counter area; above the decode-phase row limit the
    workspace holds the rotated activations (M x IC fp16)."""
    sizes = {M: exl3.linear_workspace_bytes(M, 4096, 14336) for M in (1, 8, 16, 17, 64)}
    assert all(s % 256 == 0 and s >= 16384 for s in sizes.values())
    for M in (17, 64):
        assert sizes[M] >= 16384 + M * 4096 * 2
    assert exl3.linear_workspace_bytes(0, 4096, 14336) >= 16384


def test_multi_rejects_bad_shard():
    sh = (exl3.Shard * 2)()
    sh[0] = exl3.Shard(FAKE, 256, 2, 0, 0, FAKE, FAKE, FAKE, FAKE)
    sh[1] = exl3.Shard(FAKE, 256, 3, 0, 200, FAKE, FAKE, FAKE, FAKE)      # overlaps past ldo=400
    rc = exl3.lib().exl3_linear_multi_into(FAKE, 400, FAKE, 4, 512, 2, sh, 0, None, 0, None)
    assert rc == exl3.EINVAL and "shards[1].col0" in exl3.last_error()
    rc = exl3.lib().exl3_linear_multi_into(FAKE, 512, FAKE, 4, 512, 0, sh, 0, None, 0, None)
    assert rc == exl3.EINVAL and "n_shards" in exl3.last_error()


def test_decode_tiles_rejects():
    L = exl3.lib()
    assert L.exl3_decode_tiles(FAKE, FAKE, 100, 32, 2, None) == exl3.EINVAL
    assert L.exl3_decode_tiles(FAKE, FAKE, 32, 32, 0, None) == exl3.EINVAL
    assert L.exl3_decode_tiles(FAKE, FAKE + 8, 32, 32, 2, None) == exl3.EINVAL


def test_rotate_rejects():
    L = exl3.lib()
    assert L.exl3_rotate_activations(FAKE, None, FAKE, 4, 100, FAKE, FAKE, 0, None) == exl3.EINVAL
    assert L.exl3_rotate_activations(FAKE, None, FAKE, 4, 128, FAKE, FAKE, exl3.ACT_INT8, None) == exl3.EINVAL
    assert L.exl3_rotate_activations(FAKE, None, FAKE, 0, 128, FAKE, FAKE, 0, None) == exl3.OK


def test_gemm_split_plan():
    """The K split fills about 1024 one-wave tiles, keeps >= 8 steps (512 features) per split, is 1 once
    the shard has 1024 tiles, and the workspace holds the partial tiles."""
    L = exl3.lib()
    for M, IC, OC in ((200, 2048, 256), (1, 17408, 5120), (64, 5120, 17408), (8192, 5120, 17408),
                      (1024, 4096, 14336), (129, 512, 128), (300, 1536, 384)):
        s = L.exl3_gemm_splits(M, IC, OC)
        tiles = -(-M // 128) * (OC // 128)
        assert 1 <= s <= max(1, (IC // 64) // 8)
        assert s == 1 or s * tiles <= 1024
        if tiles >= 1024:
            assert s == 1
        if s > 1 and M > L.exl3_gemv_max_rows(OC):
            assert exl3.linear_workspace_bytes(M, IC, OC) >= s * tiles * 65536 + M * IC * 2
    assert L.exl3_gemm_splits(200, 2048, 256) == 4
    assert L.exl3_gemm_splits(0, 2048, 256) == 1 and L.exl3_gemm_splits(4, 100, 256) == 1


def test_lm_head_validation():
    """Host-side checks of the output head (no launch): H a positive multiple of 64, ldo >= V, M >= 0, non-null and aligned pointers; M == 0 is a no-op."""
    L = exl3.lib()
    f = L.exl3_lm_head_int8
    assert f(FAKE, 100, FAKE, 2, FAKE, FAKE, 100, 96, None) == exl3.EINVAL and "H" in exl3.last_error()
    assert f(FAKE, 99, FAKE, 2, FAKE, FAKE, 100, 128, None) == exl3.EINVAL and "ldo" in exl3.last_error()
    assert f(FAKE, 100, FAKE, -1, FAKE, FAKE, 100, 128, None) == exl3.EINVAL and "M" in exl3.last_error()
    assert f(FAKE, 100, FAKE, 2, FAKE, FAKE, 0, 128, None) == exl3.EINVAL and "V" in exl3.last_error()
    assert f(FAKE, 100, None, 2, FAKE, FAKE, 100, 128, None) == exl3.EINVAL and "null" in exl3.last_error()
    assert f(FAKE, 100, FAKE + 8, 2, FAKE, FAKE, 100, 128, None) == exl3.EINVAL and "aligned" in exl3.last_error()
    assert f(FAKE + 1, 100, FAKE, 2, FAKE, FAKE, 100, 128, None) == exl3.EINVAL and "aligned" in exl3.last_error()
    assert f(None, 100, None, 0, None, None, 100, 128, None) == exl3.OK


def test_mlp_validation():
    """Host-side checks of the dense MLP block (no launch)."""
    L = exl3.lib()
    g = exl3.Shard(FAKE, 256, 2, 0, 0, FAKE, FAKE, FAKE, FAKE)
    d = exl3.Shard(FAKE, 128, 3, 0, 0, FAKE, FAKE, FAKE, FAKE)
    call = lambda M, H, I, gate, up, down, ws=FAKE, nb=1 << 30: L.exl3_mlp_forward(
        FAKE, FAKE, M, H, I, ctypes.byref(gate), ctypes.byref(up), ctypes.byref(down), 0, ws, nb, None)
    assert call(2, 100, 256, g, g, d) == exl3.EINVAL and "H" in exl3.last_error()
    assert call(2, 128, 200, g, g, d) == exl3.EINVAL and "I" in exl3.last_error()
    assert call(2, 128, 256, g, d, d) == exl3.EINVAL and "OC" in exl3.last_error()
    assert call(2, 128, 256, g, g, g) == exl3.EINVAL and "down" in exl3.last_error()
    assert call(2, 128, 256, g, g, d, ws=None) == exl3.EWORKSPACE
    need = L.exl3_mlp_workspace_bytes(2, 128, 256, ctypes.byref(g), ctypes.byref(g), 0)
    assert need >= 16384 + 2 * 512 * 2 + 2 * 256 * 2 and need % 256 == 0
    assert call(2, 128, 256, g, g, d, nb=need - 1) == exl3.EWORKSPACE and "ws_bytes" in exl3.last_error()
    assert call(0, 128, 256, g, g, d) == exl3.OK
    assert L.exl3_silu_mul(FAKE, FAKE, 2, 12, None) == exl3.EINVAL
    assert L.exl3_silu_mul(None, None, 0, 16, None) == exl3.OK


def test_missing_library_fails_loudly(monkeypatch):
    """No fallback: without the built library every entry point raises before doing anything."""
    import torch
    monkeypatch.setattr(exl3, "_lib", None)
    monkeypatch.setattr(exl3, "LIB_PATH", os.path.join(ROOT, "no_such_dir", "libexl3.so"))
    with pytest.raises(RuntimeError, match="not built"):
        exl3.lib()
    table = torch.zeros((4, 16), dtype=torch.int8)
    scale = torch.zeros((4,), dtype=torch.bfloat16)
    with pytest.raises(RuntimeError, match="not built"):
        exl3.embed_int8(table, scale, torch.zeros((2,), dtype=torch.int32))
    with pytest.raises(RuntimeError, match="not built"):
        exl3.linear_workspace_bytes(4, 512, 512)
