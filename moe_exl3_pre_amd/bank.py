"""Host-side packing of one layer's MoE expert bank into the layout exl3_moe_bank_forward reads.

Layout ("dspark/worker/exl3/bank.py", `Exl3Bank` and `allocate`): the slot order sorts the experts by
their bit widths, so the slots of one (k_gu, k_d) pair form one contiguous run.  One int16 array holds,
slot after slot, the w1 words and then the w3 words; a second int16 array holds the w2 words the same
way.  The fp16 sign/scale vectors are indexed by slot.

Slot order: a stable sort of the logical expert ids by (k_gu, k_d), ascending; the groups are the
maximal runs of equal (k_gu, k_d).  perm[e] is the slot of logical expert e.
"""
from __future__ import annotations

import ctypes

import numpy as np


class PackedBank:
    """numpy arrays of a packed bank (slot order) plus its tables."""

    def __init__(self, E, H, I, w13, w2, w13_suh, w13_svh, w2_suh, w2_svh, off_w1, off_w3, off_w2, perm, groups,
                 k_gu, k_d):
        self.E, self.H, self.I = E, H, I
        self.w13, self.w2 = w13, w2
        self.w13_suh, self.w13_svh, self.w2_suh, self.w2_svh = w13_suh, w13_svh, w2_suh, w2_svh
        self.off_w1, self.off_w3, self.off_w2 = off_w1, off_w3, off_w2
        self.perm = perm
        self.groups = groups          # list of (k_gu, k_d, lo, hi)
        self.k_gu, self.k_d = k_gu, k_d   # per slot

    def trellis_bytes(self, slots=None) -> int:
        """Trellis words (bytes) of the given slots (all by default)."""
        slots = range(self.E) if slots is None else slots
        return sum(2 * self.H * self.I * int(self.k_gu[p]) // 8 + self.H * self.I * int(self.k_d[p]) // 8
                   for p in slots)

    def projection(self, p: int, name: str):
        """Projection `name` ("w1", "w3" or "w2") of physical slot p: (trellis words reshaped to the tile grid
        [IC/16, OC/16, 16 K] as a view of the flat bank, input sign/scale vector, output sign/scale vector,
        K).  w1 and w3 read H features and give I, w2 the other way round."""
        H, I = self.H, self.I
        if name == "w2":
            K = int(self.k_d[p])
            grid, flat, start, s_in, s_out = (I // 16, H // 16, 16 * K), self.w2, self.off_w2[p], \
                self.w2_suh[p], self.w2_svh[p]
        else:
            K = int(self.k_gu[p])
            h = {"w1": 0, "w3": 1}[name]
            start = (self.off_w1 if h == 0 else self.off_w3)[p]
            grid, flat, s_in, s_out = (H // 16, I // 16, 16 * K), self.w13, self.w13_suh[p, h], self.w13_svh[p, h]
        n = grid[0] * grid[1] * grid[2]
        return flat[start:start + n].reshape(grid), s_in, s_out, K


def pack_bank(experts, H: int, I: int) -> PackedBank:
    """Pack logical experts (dicts with w1, w3, w2 int16 trellis arrays, k_gu, k_d and the fp16 vectors
    w1_suh, w3_suh [H], w1_svh, w3_svh [I], w2_suh [I], w2_svh [H]) into slot order."""
    E = len(experts)
    keys = [(int(e["k_gu"]), int(e["k_d"])) for e in experts]
    order = sorted(range(E), key=lambda e: keys[e])          # stable
    perm = np.empty(E, dtype=np.int32)
    perm[np.asarray(order)] = np.arange(E, dtype=np.int32)
    k_gu = np.array([keys[e][0] for e in order], dtype=np.int32)
    k_d = np.array([keys[e][1] for e in order], dtype=np.int32)
    groups, lo = [], 0
    for p in range(1, E + 1):
        if p == E or keys[order[p]] != keys[order[lo]]:
            groups.append((keys[order[lo]][0], keys[order[lo]][1], lo, p))
            lo = p
    n13 = [H * I * int(k) // 16 for k in k_gu]
    n2 = [I * H * int(k) // 16 for k in k_d]
    off_w1 = np.zeros(E, dtype=np.int64)
    off_w2 = np.zeros(E, dtype=np.int64)
    acc13 = acc2 = 0
    for p in range(E):
        off_w1[p] = acc13
        acc13 += 2 * n13[p]
        off_w2[p] = acc2
        acc2 += n2[p]
    off_w3 = off_w1 + np.asarray(n13, dtype=np.int64)
    w13 = np.empty(acc13, dtype=np.int16)
    w2 = np.empty(acc2, dtype=np.int16)
    w13_suh = np.empty((E, 2, H), dtype=np.float16)
    w13_svh = np.empty((E, 2, I), dtype=np.float16)
    w2_suh = np.empty((E, I), dtype=np.float16)
    w2_svh = np.empty((E, H), dtype=np.float16)
    for p, e in enumerate(order):
        x = experts[e]
        for name, shape in (("w1", (H // 16, I // 16, 16 * k_gu[p])), ("w3", (H // 16, I // 16, 16 * k_gu[p])),
                            ("w2", (I // 16, H // 16, 16 * k_d[p]))):
            if tuple(x[name].shape) != shape or x[name].dtype != np.int16:
                raise ValueError(f"expert {e} {name}: got {tuple(x[name].shape)} {x[name].dtype}, expected {shape} int16")
        w13[off_w1[p]:off_w1[p] + n13[p]] = x["w1"].reshape(-1)
        w13[off_w3[p]:off_w3[p] + n13[p]] = x["w3"].reshape(-1)
        w2[off_w2[p]:off_w2[p] + n2[p]] = x["w2"].reshape(-1)
        w13_suh[p, 0], w13_suh[p, 1] = x["w1_suh"], x["w3_suh"]
        w13_svh[p, 0], w13_svh[p, 1] = x["w1_svh"], x["w3_svh"]
        w2_suh[p], w2_svh[p] = x["w2_suh"], x["w2_svh"]
    return PackedBank(E, H, I, w13, w2, w13_suh, w13_svh, w2_suh, w2_svh, off_w1, off_w3, off_w2, perm, groups,
                      k_gu, k_d)


class DeviceBank:
    """A packed bank resident on one GPU, with the exl3_bank descriptor that points into it."""

    def __init__(self, packed: PackedBank, device):
        import torch
        from . import exl3
        self.packed = packed
        to = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
        self.E, self.H, self.I = packed.E, packed.H, packed.I
        self.tensors = {name: to(getattr(packed, name)) for name in
                        ("w13", "w2", "w13_suh", "w13_svh", "w2_suh", "w2_svh", "off_w1", "off_w3", "off_w2", "perm")}
        n = len(packed.groups)
        self._groups = (exl3.Group * n)(*[exl3.Group(kg, kd, lo, hi) for kg, kd, lo, hi in packed.groups])
        t = self.tensors
        self.struct = exl3.Bank(packed.E, packed.H, packed.I, n, t["w13"].data_ptr(), t["w2"].data_ptr(),
                                t["w13_suh"].data_ptr(), t["w13_svh"].data_ptr(), t["w2_suh"].data_ptr(),
                                t["w2_svh"].data_ptr(), t["off_w1"].data_ptr(), t["off_w3"].data_ptr(),
                                t["off_w2"].data_ptr(), t["perm"].data_ptr(),
                                ctypes.cast(self._groups, ctypes.POINTER(exl3.Group)))
        self.device = device
