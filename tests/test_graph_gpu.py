"""The dense MLP block, the int8 output head and the embedding gather captured in a HIP graph: every replay
(with eager calls and synchronisations between replays) equals the eager result bit for bit."""
import numpy as np
import pytest
import torch

from moe_exl3_pre_amd import exl3, synth
from tests.helpers import dev, log, shard_to_dev, to_dev, to_dev_x

pytestmark = pytest.mark.gpu


def _replays_match(call, out, eager):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()                                              # warm-up outside capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    for i in range(4):
        out.fill_(float(i + 1))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i}"
        call()                                              # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(out, eager)


@pytest.mark.parametrize("M", [3, 8])
def test_mlp_graph_replay(M):
    """M=3 writes h for the in-kernel rotation; M=8 folds the activation into down's pre-pass."""
    log(f"mlp graph M={M}")
    c = synth.mlp_case(300 + M, M, 512, 1024, 2, 3, 3)
    s_in, rin = to_dev(c["gate"]["s_in"]), to_dev(c["gate"]["rin"])
    x = to_dev_x(c["x_bits"])
    g, u, d = shard_to_dev(c["gate"], s_in, rin), shard_to_dev(c["up"], s_in, rin), shard_to_dev(c["down"])
    ws = exl3.alloc_workspace(exl3.mlp_workspace_bytes(M, 512, 1024, g, u), dev())
    eager = exl3.mlp_forward(x, g, u, d, ws=ws).clone()
    torch.cuda.synchronize()
    out = torch.empty_like(eager)
    _replays_match(lambda: exl3.mlp_forward(x, g, u, d, out=out, ws=ws), out, eager)


def test_lm_head_and_embed_graph_replay():
    log("lm_head/embed graph")
    rng = np.random.default_rng(310)
    V, H, M, T = 997, 320, 5, 40
    table = torch.from_numpy(rng.integers(-128, 128, size=(V, H), dtype=np.int8)).to(dev())
    scale = torch.from_numpy(rng.integers(0x3A00, 0x3D80, size=V).astype(np.int16)).to(dev()).view(torch.bfloat16)
    x = torch.from_numpy(rng.normal(size=(M, H)).astype(np.float32)).to(dev()).to(torch.bfloat16)
    ids = torch.from_numpy(rng.integers(-2, V + 2, size=T).astype(np.int32)).to(dev())
    eager = exl3.lm_head_int8(x, table, scale).clone()
    out = torch.empty_like(eager)
    _replays_match(lambda: exl3.lm_head_int8(x, table, scale, out=out), out, eager)
    eager_e = exl3.embed_int8(table, scale, ids).clone()
    out_e = torch.empty_like(eager_e)
    _replays_match(lambda: exl3.embed_int8(table, scale, ids, out=out_e), out_e, eager_e)
