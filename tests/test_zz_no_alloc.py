"""The allocation-free entry point (exl3_linear_multi_into_static) through the C ABI: bitwise equal to
exl3_linear_multi_into with a caller workspace, over consecutive calls that share the static scratch."""
import ctypes

import numpy as np
import pytest
import torch

from moe_exl3_pre_amd import exl3, synth
from tests.helpers import dev, log, shard_to_dev, to_dev, to_dev_x

pytestmark = pytest.mark.gpu

SENTINEL = -1000.0


def _dev_merged(seed, M, IC, shards):
    case = synth.merged_case(seed, M, IC, shards)
    x = to_dev_x(case["x_bits"])
    s_in, rin = to_dev(case["shards"][0]["s_in"]), to_dev(case["shards"][0]["rin"])
    return case, x, [shard_to_dev(s, s_in, rin) for s in case["shards"]]


def _static_call(out, x, shards, flags=0):
    """Straight through the C ABI (no binding-side workspace)."""
    M, IC = x.shape
    arr = exl3._shard_array(shards)
    rc = exl3.lib().exl3_linear_multi_into_static(ctypes.c_void_p(out.data_ptr()), out.shape[1],
                                                  ctypes.c_void_p(x.data_ptr()), M, IC, len(shards), arr, flags,
                                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    return rc


def _both(case, x, shards, flags=0):
    M = x.shape[0]
    a = torch.full((M, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    exl3.linear_multi_into(a, x, shards, flags=flags)
    b = torch.full_like(a, SENTINEL)
    rc = _static_call(b, x, shards, flags)
    torch.cuda.synchronize()
    assert rc == exl3.OK, exl3.last_error()
    return a, b


def test_static_entry_equals_workspace_entry_on_consecutive_calls():
    """Three calls in a row on the one static scratch, each smaller than the one before:
    (1) the decode-phase gate_up of IC=4096, 2 x 14336 (K=2 | K=3) at M=8: split-K slab and counters, and
        the once-per-call rotation region;
    (2) the same weights at M=1 (in-block rotation; the counters must have been left at zero by call 1);
    (3) M=3 over two small shards (IC=512)."""
    L = exl3.lib()
    assert L.exl3_static_scratch_bytes() == 16 << 20
    case, x, shards = _dev_merged(4100, 8, 4096, [(14336, 2), (14336, 3)])
    for M in (8, 1):
        log(f"static entry: gate_up 4096 -> 2 x 14336, M={M}")
        a, b = _both(case, x[:M].contiguous(), shards)
        assert torch.equal(a, b), M
        assert torch.isfinite(b.float()).all()
    case2, x2, shards2 = _dev_merged(4101, 3, 512, [(256, 2), (384, 4)])
    log("static entry: IC=512, 256 | 384 columns, M=3")
    a, b = _both(case2, x2, shards2)
    assert torch.equal(a, b)
    # the first call again: the scratch still serves it (counters back at zero after every call)
    a, b = _both(case, x, shards)
    assert torch.equal(a, b)


def test_static_entry_gemm_path_within_the_limit():
    """A prefill-phase call whose workspace fits (M=40, IC=512): the feature-split GEMM's partial tiles and
    its rotated activations in the static scratch; then a smaller decode-phase call."""
    case, x, shards = _dev_merged(4102, 40, 512, [(256, 2), (384, 3)])
    need = exl3.linear_multi_workspace_bytes(40, 512, shards, exl3.FORCE_MFMA)
    assert need <= exl3.lib().exl3_static_scratch_bytes()
    log(f"static entry: GEMM path M=40, workspace {need} bytes")
    a, b = _both(case, x, shards, flags=exl3.FORCE_MFMA)
    assert torch.equal(a, b)
    a, b = _both(case, x[:2].contiguous(), shards)
    assert torch.equal(a, b)


def test_static_entry_rejects_a_call_beyond_the_scratch():
    """M=4096 rows of the gate_up need more than 16 MiB (rotated activations alone are 32 MiB): the call
    launches nothing, returns EXL3_EWORKSPACE and names the limit; the output stays untouched."""
    case, x, shards = _dev_merged(4103, 1, 4096, [(14336, 2), (14336, 3)])
    xb = x.expand(4096, 4096).contiguous()
    assert exl3.linear_multi_workspace_bytes(4096, 4096, shards) > exl3.lib().exl3_static_scratch_bytes()
    out = torch.full((4096, case["ldo"]), SENTINEL, dtype=torch.bfloat16, device=dev())
    rc = _static_call(out, xb, shards)
    torch.cuda.synchronize()
    assert rc == exl3.EWORKSPACE
    assert "static scratch holds" in exl3.last_error()
    assert torch.all(out == SENTINEL)
