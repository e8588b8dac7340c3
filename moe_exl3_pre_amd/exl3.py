"""Thin Python binding of the EXL3 C ABI (include/exl3.h).

Argument marshalling only: tensors are checked for dtype, shape, device and contiguity, and their
data pointers and the current HIP stream are handed to the library.  Every step of the layer runs in
the HIP kernels of libexl3.so; there is no fallback path.  If the library is missing, every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libexl3.so")

OK, EINVAL, EWORKSPACE, EUNSUPPORTED, ELAUNCH = 0, -1, -2, -3, -4
ACT_INT8, FORCE_GEMV, FORCE_MFMA, GEMM_NO_SPLIT, BATCH_INVARIANT = 1, 2, 4, 8, 16

_lib = None


class Exl3Error(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"exl3 status {status}: {message}")
        self.status = status


class Shard(ctypes.Structure):
    _fields_ = [("code", ctypes.c_void_p), ("OC", ctypes.c_int64), ("K", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("col0", ctypes.c_int64), ("s_in", ctypes.c_void_p), ("rin", ctypes.c_void_p),
                ("rout", ctypes.c_void_p), ("s_out", ctypes.c_void_p)]


class Group(ctypes.Structure):
    _fields_ = [("k_gu", ctypes.c_int32), ("k_d", ctypes.c_int32), ("lo", ctypes.c_int32), ("hi", ctypes.c_int32)]


class Bank(ctypes.Structure):
    _fields_ = [("E", ctypes.c_int32), ("H", ctypes.c_int32), ("I", ctypes.c_int32), ("n_groups", ctypes.c_int32),
                ("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("w13_suh", ctypes.c_void_p), ("w13_svh", ctypes.c_void_p),
                ("w2_suh", ctypes.c_void_p), ("w2_svh", ctypes.c_void_p),
                ("off_w1", ctypes.c_void_p), ("off_w3", ctypes.c_void_p), ("off_w2", ctypes.c_void_p),
                ("perm", ctypes.c_void_p), ("groups", ctypes.POINTER(Group))]


# name -> (restype, argtypes); mirrors include/exl3.h
_SIGS = {
    "exl3_last_error": (ctypes.c_char_p, []),
    "exl3_version": (ctypes.c_int, []),
    "exl3_gemv_max_rows": (ctypes.c_int64, [ctypes.c_int64]),
    "exl3_gemm_splits": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
    "exl3_gemm_tail_splits": (ctypes.c_int, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]),
    "exl3_linear_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint]),
    "exl3_linear_into": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint,
                                        ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "exl3_linear_multi_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                                            ctypes.POINTER(Shard), ctypes.c_uint]),
    "exl3_linear_multi_into": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                              ctypes.c_int64, ctypes.c_int, ctypes.POINTER(Shard), ctypes.c_uint,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "exl3_probe_read": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                       ctypes.c_void_p]),
    "exl3_probe_mfma": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]),
    "exl3_static_scratch_bytes": (ctypes.c_size_t, []),
    "exl3_linear_multi_into_static": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                                     ctypes.c_int64, ctypes.c_int, ctypes.POINTER(Shard), ctypes.c_uint,
                                                     ctypes.c_void_p]),
    "exl3_moe_workspace_bytes": (ctypes.c_size_t, [ctypes.POINTER(Bank), ctypes.c_int64, ctypes.c_int, ctypes.c_uint]),
    "exl3_moe_bank_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int, ctypes.POINTER(Bank), ctypes.c_uint,
                                             ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "exl3_lm_head_int8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64,
                                         ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_void_p]),
    "exl3_mlp_workspace_bytes": (ctypes.c_size_t, [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                                                  ctypes.POINTER(Shard), ctypes.POINTER(Shard), ctypes.c_uint]),
    "exl3_mlp_forward": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                        ctypes.c_int64, ctypes.POINTER(Shard), ctypes.POINTER(Shard),
                                        ctypes.POINTER(Shard), ctypes.c_uint, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_void_p]),
    "exl3_silu_mul": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_void_p]),
    "exl3_embed_int8": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64,
                                       ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]),
    "exl3_decode_tiles": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int,
                                         ctypes.c_void_p]),
    "exl3_rotate_activations": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_uint,
                                               ctypes.c_void_p]),
}


def lib() -> ctypes.CDLL:
    """The loaded library.  Raises if it has not been built: there is no other implementation."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"EXL3 HIP library not built ({LIB_PATH} missing): run `python -m moe_exl3_pre_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(h, name)
            fn.restype, fn.argtypes = res, args
        _lib = h
    return _lib


def exported_symbols() -> list[str]:
    return list(_SIGS)


def last_error() -> str:
    return lib().exl3_last_error().decode()


def _check(rc: int):
    if rc != OK:
        raise Exl3Error(rc, last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtype, shape=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name}: on {t.device}, expected {device}")


# ------------------------------------------------------------------------------------------ workspace

def linear_workspace_bytes(M: int, IC: int, OC: int, flags: int = 0) -> int:
    return int(lib().exl3_linear_workspace_bytes(M, IC, OC, flags))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """A zero-filled workspace (the ABI wants it zeroed once; kernels leave their counters at zero)."""
    return torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# ------------------------------------------------------------------------------------------ linear

def linear_into(out, x, code, K, s_in, rin, rout, s_out, col0: int = 0, flags: int = 0, ws=None):
    """out[:, col0:col0+OC] = EXL3 projection of x (bf16 [M, IC]); see exl3_linear_into."""
    dev = x.device
    M, IC = x.shape
    _need(x, "x", torch.bfloat16, device=dev)
    _need(code, "code", torch.int16, device=dev)
    if code.dim() != 3 or code.shape[0] * 16 != IC or code.shape[2] != 16 * K:
        raise ValueError(f"code: shape {tuple(code.shape)} does not match IC={IC}, K={K}")
    OC = code.shape[1] * 16
    _need(out, "out", torch.bfloat16, device=dev)
    if out.dim() != 2 or out.shape[0] != M:
        raise ValueError(f"out: shape {tuple(out.shape)} does not have M={M} rows")
    for name, t, n in (("s_in", s_in, IC), ("rin", rin, IC), ("rout", rout, OC), ("s_out", s_out, OC)):
        _need(t, name, torch.float16, (n,), dev)
    if ws is None:
        ws = alloc_workspace(linear_workspace_bytes(M, IC, OC, flags), dev)
    _check(lib().exl3_linear_into(_ptr(out), out.shape[1], col0, _ptr(x), M, IC, _ptr(code), OC, K, _ptr(s_in),
                                  _ptr(rin), _ptr(rout), _ptr(s_out), flags, _ptr(ws), ws.numel(), _stream(dev)))
    return out


def _shard_array(shards):
    arr = (Shard * len(shards))()
    for i, s in enumerate(shards):
        arr[i] = Shard(_ptr(s["code"]), s["code"].shape[1] * 16, s["K"], 0, s["col0"], _ptr(s["s_in"]), _ptr(s["rin"]),
                       _ptr(s["rout"]), _ptr(s["s_out"]))
    return arr


def linear_multi_workspace_bytes(M: int, IC: int, shards, flags: int = 0) -> int:
    arr = _shard_array(shards)
    return int(lib().exl3_linear_multi_workspace_bytes(M, IC, len(shards), arr, flags))


def linear_multi_into(out, x, shards, flags: int = 0, ws=None):
    """Several shards (dicts with code, K, col0, s_in, rin, rout, s_out) into their column slices of out."""
    dev = x.device
    M, IC = x.shape
    _need(x, "x", torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, device=dev)
    for i, s in enumerate(shards):
        _need(s["code"], f"shards[{i}].code", torch.int16, device=dev)
        if s["code"].shape[0] * 16 != IC or s["code"].shape[2] != 16 * s["K"]:
            raise ValueError(f"shards[{i}].code: shape {tuple(s['code'].shape)} does not match IC={IC}, K={s['K']}")
        OC = s["code"].shape[1] * 16
        for name, n in (("s_in", IC), ("rin", IC), ("rout", OC), ("s_out", OC)):
            _need(s[name], f"shards[{i}].{name}", torch.float16, (n,), dev)
    arr = _shard_array(shards)
    if ws is None:
        ws = alloc_workspace(lib().exl3_linear_multi_workspace_bytes(M, IC, len(shards), arr, flags), dev)
    _check(lib().exl3_linear_multi_into(_ptr(out), out.shape[1], _ptr(x), M, IC, len(shards), arr, flags, _ptr(ws),
                                        ws.numel(), _stream(dev)))
    return out


def linear_multi_into_static(out, x, shards, flags: int = 0):
    """exl3_linear_multi_into with the library's static device scratch as its workspace (no allocation);
    see exl3_linear_multi_into_static for the size limit and the sharing rule."""
    dev = x.device
    M, IC = x.shape
    _need(x, "x", torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, device=dev)
    for i, s in enumerate(shards):
        _need(s["code"], f"shards[{i}].code", torch.int16, device=dev)
        if s["code"].shape[0] * 16 != IC or s["code"].shape[2] != 16 * s["K"]:
            raise ValueError(f"shards[{i}].code: shape {tuple(s['code'].shape)} does not match IC={IC}, K={s['K']}")
        OC = s["code"].shape[1] * 16
        for name, n in (("s_in", IC), ("rin", IC), ("rout", OC), ("s_out", OC)):
            _need(s[name], f"shards[{i}].{name}", torch.float16, (n,), dev)
    arr = _shard_array(shards)
    _check(lib().exl3_linear_multi_into_static(_ptr(out), out.shape[1], _ptr(x), M, IC, len(shards), arr, flags,
                                               _stream(dev)))
    return out


def probe_read(src, sink, blocks: int, variant: int = 0):
    """Measurement hook: one streaming read of the bytes of `src` (device tensor, contiguous, 16-byte multiple);
    sink uint32-sized tensor of `blocks` elements.  See exl3_probe_read."""
    _check(lib().exl3_probe_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink), blocks, variant,
                                 _stream(src.device)))


def probe_mfma(sink, kind: int, iters: int, blocks: int):
    """Measurement hook: back-to-back MFMAs (kind 0 f16 16x16x32, 1 f16 32x32x16, 2 i8 16x16x64, 3 i8 32x32x32);
    sink float32 [blocks * 256].  Returns the FLOP (or OP) count of the call.  See exl3_probe_mfma."""
    _check(lib().exl3_probe_mfma(_ptr(sink), kind, iters, blocks, _stream(sink.device)))
    per = {0: 131072, 1: 131072, 2: 262144, 3: 262144}[kind]
    return float(blocks) * 4 * iters * per


# ------------------------------------------------------------------------------------------ dense MLP block

def _one_shard(s, IC, dev, name):
    _need(s["code"], f"{name}.code", torch.int16, device=dev)
    if s["code"].dim() != 3 or s["code"].shape[0] * 16 != IC or s["code"].shape[2] != 16 * s["K"]:
        raise ValueError(f"{name}.code: shape {tuple(s['code'].shape)} does not match IC={IC}, K={s['K']}")
    OC = s["code"].shape[1] * 16
    for key, n in (("s_in", IC), ("rin", IC), ("rout", OC), ("s_out", OC)):
        _need(s[key], f"{name}.{key}", torch.float16, (n,), dev)
    return Shard(_ptr(s["code"]), OC, s["K"], 0, 0, _ptr(s["s_in"]), _ptr(s["rin"]), _ptr(s["rout"]), _ptr(s["s_out"]))


def mlp_workspace_bytes(M: int, H: int, I: int, gate, up, flags: int = 0) -> int:
    g, u = _one_shard(gate, H, gate["code"].device, "gate"), _one_shard(up, H, up["code"].device, "up")
    return int(lib().exl3_mlp_workspace_bytes(M, H, I, ctypes.byref(g), ctypes.byref(u), flags))


def mlp_forward(x, gate, up, down, out=None, flags: int = 0, ws=None):
    """Dense MLP block: down(bf16(silu(gate(x)) * up(x))) for x bf16 [M, H]; gate, up and down are dicts with
    code, K, s_in, rin, rout, s_out (gate and up over H -> I, down over I -> H).  See exl3_mlp_forward."""
    dev = x.device
    _need(x, "x", torch.bfloat16, device=dev)
    M, H = x.shape
    g, u = _one_shard(gate, H, dev, "gate"), _one_shard(up, H, dev, "up")
    I = g.OC
    d = _one_shard(down, I, dev, "down")
    if out is None:
        out = torch.empty((M, H), dtype=torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (M, H), dev)
    if ws is None:
        ws = alloc_workspace(lib().exl3_mlp_workspace_bytes(M, H, I, ctypes.byref(g), ctypes.byref(u), flags), dev)
    _check(lib().exl3_mlp_forward(_ptr(out), _ptr(x), M, H, I, ctypes.byref(g), ctypes.byref(u), ctypes.byref(d),
                                  flags, _ptr(ws), ws.numel(), _stream(dev)))
    return out


def silu_mul(gu, out=None):
    """bf16 [M, I] = bf16(silu(gu[:, :I]) * gu[:, I:]) of a bf16 [M, 2I] tensor; see exl3_silu_mul."""
    _need(gu, "gu", torch.bfloat16)
    M, I2 = gu.shape
    if I2 % 2:
        raise ValueError(f"gu: {I2} columns, want 2I")
    if out is None:
        out = torch.empty((M, I2 // 2), dtype=torch.bfloat16, device=gu.device)
    _need(out, "out", torch.bfloat16, (M, I2 // 2), gu.device)
    _check(lib().exl3_silu_mul(_ptr(out), _ptr(gu), M, I2 // 2, _stream(gu.device)))
    return out


# ------------------------------------------------------------------------------------------ test hooks

def embed_int8(table, scale, ids, out=None):
    """bf16 [T, H] rows table[ids] * scale[ids] of an int8 [V, H] table with bf16 [V] row scales; ids int32 [T]."""
    _need(table, "table", torch.int8)
    _need(scale, "scale", torch.bfloat16)
    _need(ids, "ids", torch.int32)
    V, H = table.shape
    if scale.shape != (V,):
        raise ValueError(f"scale: shape {tuple(scale.shape)} != ({V},)")
    if ids.dim() != 1:
        raise ValueError(f"ids: {ids.dim()}-d, want [T]")
    T = ids.shape[0]
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=table.device)
    _need(out, "out", torch.bfloat16)
    if out.shape != (T, H):
        raise ValueError(f"out: shape {tuple(out.shape)} != ({T}, {H})")
    _check(lib().exl3_embed_int8(_ptr(out), _ptr(table), _ptr(scale), V, H, _ptr(ids), T, _stream(table.device)))
    return out


def lm_head_int8(x, table, scale, out=None):
    """bf16 logits [M, V] = x [M, H] . bf16(table * scale)^T for an int8 [V, H] table with bf16 [V] row
    scales; `out` may be a wider [M, ldo] buffer's leading V columns."""
    _need(x, "x", torch.bfloat16)
    _need(table, "table", torch.int8)
    _need(scale, "scale", torch.bfloat16)
    V, H = table.shape
    if scale.shape != (V,):
        raise ValueError(f"scale: shape {tuple(scale.shape)} != ({V},)")
    if x.dim() != 2 or x.shape[1] != H:
        raise ValueError(f"x: shape {tuple(x.shape)}, want [M, {H}]")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, V), dtype=torch.bfloat16, device=x.device)
    if out.dtype != torch.bfloat16 or out.dim() != 2 or out.shape != (M, V) or out.stride(1) != 1:
        raise ValueError(f"out: want bf16 [{M}, {V}] with unit column stride")
    _check(lib().exl3_lm_head_int8(_ptr(out), out.stride(0), _ptr(x), M, _ptr(table), _ptr(scale), V, H,
                                   _stream(x.device)))
    return out


def decode_tiles(code, K):
    """Decoded weight fp16 [IC, OC] through the device decode routine."""
    IC, OC = code.shape[0] * 16, code.shape[1] * 16
    _need(code, "code", torch.int16)
    w = torch.empty((IC, OC), dtype=torch.float16, device=code.device)
    _check(lib().exl3_decode_tiles(_ptr(w), _ptr(code), IC, OC, K, _stream(code.device)))
    return w


def rotate_activations(x, s_in, rin, int8: bool = False):
    """The pre-pass output: fp16 [M, IC], or (int8 [M, IC], float32 [M]) with int8=True."""
    M, IC = x.shape
    _need(x, "x", torch.bfloat16)
    q = torch.empty((M, IC), dtype=torch.int8 if int8 else torch.float16, device=x.device)
    sc = torch.empty((M,), dtype=torch.float32, device=x.device) if int8 else None
    _check(lib().exl3_rotate_activations(_ptr(q), _ptr(sc), _ptr(x), M, IC, _ptr(s_in), _ptr(rin),
                                         ACT_INT8 if int8 else 0, _stream(x.device)))
    return (q, sc) if int8 else q


# ------------------------------------------------------------------------------------------ MoE bank

def moe_workspace_bytes(bank, T: int, topk: int, flags: int = 0) -> int:
    return int(lib().exl3_moe_workspace_bytes(ctypes.byref(bank.struct), T, topk, flags))


def moe_bank_forward(out, x, topk_ids, topk_w, bank, flags: int = 0, ws=None):
    """out = sum_j topk_w[:, j] * expert_{topk_ids[:, j]}(x) for a DeviceBank; see exl3_moe_bank_forward."""
    dev = x.device
    T, H = x.shape
    if H != bank.H:
        raise ValueError(f"x: hidden size {H} does not match the bank's {bank.H}")
    _need(x, "x", torch.bfloat16, device=dev)
    _need(out, "out", torch.bfloat16, (T, H), dev)
    if topk_ids.dim() != 2 or topk_ids.shape[0] != T:
        raise ValueError(f"topk_ids: shape {tuple(topk_ids.shape)} does not have T={T} rows")
    topk = topk_ids.shape[1]
    _need(topk_ids, "topk_ids", torch.int32, (T, topk), dev)
    _need(topk_w, "topk_w", torch.float32, (T, topk), dev)
    if ws is None:
        ws = alloc_workspace(moe_workspace_bytes(bank, T, topk, flags), dev)
    _check(lib().exl3_moe_bank_forward(_ptr(out), _ptr(x), T, _ptr(topk_ids), _ptr(topk_w), topk,
                                       ctypes.byref(bank.struct), flags, _ptr(ws), ws.numel(), _stream(dev)))
    return out
