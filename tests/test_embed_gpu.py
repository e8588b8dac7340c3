"""GPU parity of the int8 embedding gather-dequant against the oracle, bit for bit, through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import exl3_oracle as O
from moe_exl3_pre_amd import exl3
from tests.helpers import dev, log

pytestmark = pytest.mark.gpu


def _case(seed, V, H):
    rng = np.random.default_rng(seed)
    table = rng.integers(-128, 128, size=(V, H), dtype=np.int8)
    scale = rng.integers(0x3A00, 0x3D80, size=V).astype(np.uint16)      # bf16 ~ 4.9e-4 .. 6.2e-2
    scale[rng.random(V) < 0.25] |= 0x8000                                # some negative scales
    return rng, table, scale


def _run(table, scale, ids):
    t = torch.from_numpy(table).to(dev())
    s = torch.from_numpy(scale.view(np.int16)).to(dev()).view(torch.bfloat16)
    i = torch.from_numpy(np.asarray(ids, dtype=np.int32)).to(dev())
    out = exl3.embed_int8(t, s, i)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16)


def test_embed_bit_exact_with_invalid_and_repeated_ids():
    """H = 5168: five full 1024-column wave chunks and a 48-column one (three lanes)."""
    V, H, T = 1000, 5168, 300
    rng, table, scale = _case(21, V, H)
    ids = rng.integers(0, V, size=T)
    ids[[3, 50, 299]] = [-1, V, 1 << 30]                                 # out of range: zero rows
    ids[100:110] = ids[0]                                                # repeats
    log(f"embed V={V} H={H} T={T}")
    assert np.array_equal(_run(table, scale, ids), O.embed_gather(table, scale, ids))


@pytest.mark.parametrize("H,T", [(16, 7), (1024, 1), (2048, 65)])
def test_embed_shapes(H, T):
    V = 97
    rng, table, scale = _case(22 + H + T, V, H)
    ids = rng.integers(-5, V + 5, size=T)
    assert np.array_equal(_run(table, scale, ids), O.embed_gather(table, scale, ids))


def test_embed_zero_tokens_is_a_no_op():
    _, table, scale = _case(23, 10, 64)
    t = torch.from_numpy(table).to(dev())
    s = torch.from_numpy(scale.view(np.int16)).to(dev()).view(torch.bfloat16)
    out = torch.full((0, 64), 1.0, dtype=torch.bfloat16, device=dev())
    exl3.embed_int8(t, s, torch.empty((0,), dtype=torch.int32, device=dev()), out=out)
    torch.cuda.synchronize()


def test_embed_full_vocabulary_sampled():
    """The pages' vocabulary: 248,320 rows of 5120 (a 1.27 GB int8 table); 512 random ids checked against the
    oracle on the gathered rows."""
    V, H, T = 248320, 5120, 512
    g = torch.Generator(device=dev())
    g.manual_seed(24)
    table = torch.randint(-128, 128, (V, H), dtype=torch.int8, device=dev(), generator=g)
    scale = torch.randint(0x3A00, 0x3D80, (V,), dtype=torch.int32, device=dev(), generator=g).to(torch.int16)
    scale = scale.view(torch.bfloat16)
    ids = torch.randint(0, V, (T,), dtype=torch.int32, device=dev(), generator=g)
    ids[-1] = V - 1
    log(f"embed full vocabulary V={V} H={H} T={T}")
    out = exl3.embed_int8(table, scale, ids)
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    rows = table[ids.long()].cpu().numpy()
    srows = scale[ids.long()].view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, O.embed_gather(rows, srows, np.arange(T)))
    del table
    torch.cuda.empty_cache()
