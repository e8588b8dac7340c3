"""GPU parity of the int8 output head (x . bf16(table * scale)^T) against the oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from oracle import exl3_oracle as O
from moe_exl3_pre_amd import exl3
from tests.helpers import dev, log

pytestmark = pytest.mark.gpu


def _table(seed, V, H):
    rng = np.random.default_rng(seed)
    table = rng.integers(-128, 128, size=(V, H), dtype=np.int8)
    scale = rng.integers(0x3A00, 0x3D80, size=V).astype(np.uint16)      # bf16 ~ 4.9e-4 .. 6.2e-2
    scale[rng.random(V) < 0.25] |= 0x8000
    return rng, table, scale


def _bf16_bits(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_dev(bits, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev()).view(dtype)


def _bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _check(got_bits, x_bits, table, scale):
    """Within one bf16 rounding of the exact sum: |d| <= 2^-7 |ref| + 2^-16 sum_h |x w| (the fp32 sum's
    rounding under cancellation); at least 99% of the logits bit-equal."""
    ref_bits = O.lm_head_int8(x_bits, table, scale)
    ref, got = O.bf16_bits_to_f64(ref_bits), O.bf16_bits_to_f64(got_bits)
    w = O.bf16_bits_to_f64(O.f64_to_bf16_bits(table.astype(np.float64) * O.bf16_bits_to_f64(scale)[:, None]))
    mag = np.abs(O.bf16_bits_to_f64(x_bits)) @ np.abs(w).T
    bad = np.abs(got - ref) > 2.0 ** -7 * np.abs(ref) + 2.0 ** -16 * mag
    assert not bad.any(), (np.argwhere(bad)[:5], got[bad][:5], ref[bad][:5])
    assert np.mean(got_bits == ref_bits) >= 0.99


@pytest.mark.parametrize("M", [1, 5, 16, 17, 40, 64, 65, 130])
def test_lm_head_rows(M):
    """Every 16-row group count (1..4 per launch) and several launches; V = 997 leaves a partial wave and a
    partial 4-row store; H = 320 runs one 4-step batch and one single step."""
    V, H = 997, 320
    rng, table, scale = _table(40 + M, V, H)
    x = _bf16_bits(rng.normal(size=(M, H)))
    log(f"lm_head V={V} H={H} M={M}")
    out = exl3.lm_head_int8(_to_dev(x), _to_dev(table, torch.int8), _to_dev(scale))
    torch.cuda.synchronize()
    _check(_bits(out), x, table, scale)


@pytest.mark.parametrize("M", [3, 7, 12, 30])
def test_lm_head_batched_steps(M):
    """H = 2112 is 33 feature steps: parts of 8, 8, 8 and 9 steps, so the batched loads and the single-step
    tail both run in every row-group configuration."""
    V, H = 997, 2112
    rng, table, scale = _table(60 + M, V, H)
    x = _bf16_bits(rng.normal(size=(M, H)))
    log(f"lm_head V={V} H={H} M={M}")
    out = exl3.lm_head_int8(_to_dev(x), _to_dev(table, torch.int8), _to_dev(scale))
    torch.cuda.synchronize()
    _check(_bits(out), x, table, scale)


def test_lm_head_batch_invariant():
    """A row's logits do not depend on the other rows in the call: the summation order depends only on H,
    whatever row-group configuration the call's M selects."""
    V, H = 997, 2112
    rng, table, scale = _table(70, V, H)
    x = _to_dev(_bf16_bits(rng.normal(size=(70, H))))
    t, s = _to_dev(table, torch.int8), _to_dev(scale)
    full = _bits(exl3.lm_head_int8(x, t, s))
    for M in (1, 4, 6, 9, 17, 33, 49):
        part = _bits(exl3.lm_head_int8(x[:M].contiguous(), t, s))
        assert np.array_equal(part, full[:M]), M


@pytest.mark.parametrize("M", [5, 11, 16])
def test_lm_head_x_staged_in_lds(M):
    """5..16 rows with H a multiple of 256 take the kernel that stages x in LDS; H = 1280 puts quarter
    boundaries (every 5 steps) inside its 256-feature slices."""
    V, H = 997, 1280
    rng, table, scale = _table(90 + M, V, H)
    x = _bf16_bits(rng.normal(size=(M, H)))
    log(f"lm_head staged x V={V} H={H} M={M}")
    out = exl3.lm_head_int8(_to_dev(x), _to_dev(table, torch.int8), _to_dev(scale))
    torch.cuda.synchronize()
    _check(_bits(out), x, table, scale)


def test_lm_head_batch_invariant_across_kernels():
    """H = 1280: rows 0..63 of a 70-row call run on the 64-row kernel and rows 64..69 on the staged-x
    kernel; calls of 1..40 rows take every kernel; a row's logits are the same bits in all of them."""
    V, H = 997, 1280
    rng, table, scale = _table(99, V, H)
    x = _to_dev(_bf16_bits(rng.normal(size=(70, H))))
    t, s = _to_dev(table, torch.int8), _to_dev(scale)
    full = _bits(exl3.lm_head_int8(x, t, s))
    for M in (1, 4, 5, 9, 16, 17, 40):
        part = _bits(exl3.lm_head_int8(x[:M].contiguous(), t, s))
        assert np.array_equal(part, full[:M]), M
    tail = _bits(exl3.lm_head_int8(x[64:].contiguous(), t, s))
    assert np.array_equal(tail, full[64:])


@pytest.mark.parametrize("M", [3, 9])
def test_lm_head_vector_stores_with_ragged_tail(M):
    """ldo = 1000 (a multiple of 4) with V = 997: 8-byte stores everywhere but the last 4-column group, which
    is written element by element; columns past V stay untouched.  M = 3 runs the 16-row kernel, M = 9 the
    staged-x kernel (H = 1280)."""
    V, H, ldo = 997, 1280, 1000
    rng, table, scale = _table(110 + M, V, H)
    x = _bf16_bits(rng.normal(size=(M, H)))
    buf = torch.full((M, ldo), -7.0, dtype=torch.bfloat16, device=dev())
    exl3.lm_head_int8(_to_dev(x), _to_dev(table, torch.int8), _to_dev(scale), out=buf[:, :V])
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:, V:] == -7.0)
    _check(_bits(b[:, :V].contiguous()), x, table, scale)


def test_lm_head_strided_output_keeps_other_columns():
    V, H, M, ldo = 96, 128, 3, 132
    rng, table, scale = _table(50, V, H)
    x = _bf16_bits(rng.normal(size=(M, H)))
    buf = torch.full((M, ldo), -7.0, dtype=torch.bfloat16, device=dev())
    exl3.lm_head_int8(_to_dev(x), _to_dev(table, torch.int8), _to_dev(scale), out=buf[:, :V])
    torch.cuda.synchronize()
    b = buf.cpu()
    assert torch.all(b[:, V:] == -7.0)
    _check(_bits(b[:, :V].contiguous()), x, table, scale)


def test_lm_head_identity_rows_equal_the_embedding_gather():
    """With x the identity each logit is a single weight, so the head's weights must equal, bit for bit,
    what the embedding kernel gathers for every row, except the sign of a zero: a code 0 under a negative
    scale is -0 as a gathered value, but as a logit it is the sum 1 * (-0) + 0 * w + ... = +0."""
    V, H = 200, 64
    _, table, scale = _table(51, V, H)
    t, s = _to_dev(table, torch.int8), _to_dev(scale)
    eye = torch.eye(H, dtype=torch.bfloat16, device=dev())
    logits = exl3.lm_head_int8(eye, t, s)
    rows = exl3.embed_int8(t, s, torch.arange(V, dtype=torch.int32, device=dev()))
    torch.cuda.synchronize()
    a, b = _bits(logits).T, _bits(rows)
    diff = a != b
    assert np.all((a[diff] & 0x7FFF) == 0) and np.all((b[diff] & 0x7FFF) == 0), (a[diff][:8], b[diff][:8])
    assert diff.mean() < 0.01


def test_lm_head_zero_rows_is_a_no_op():
    _, table, scale = _table(52, 32, 64)
    out = exl3.lm_head_int8(torch.empty((0, 64), dtype=torch.bfloat16, device=dev()), _to_dev(table, torch.int8),
                            _to_dev(scale))
    torch.cuda.synchronize()
    assert out.shape == (0, 32)


@pytest.mark.parametrize("M", [1, 16])
def test_lm_head_full_vocabulary_sampled(M):
    """The pages' vocabulary (248,320 x 5120, 1.27 GB int8) at decode sizes; 256 random table rows and the
    last one checked against the oracle."""
    V, H = 248320, 5120
    g = torch.Generator(device=dev())
    g.manual_seed(53 + M)
    table = torch.randint(-128, 128, (V, H), dtype=torch.int8, device=dev(), generator=g)
    scale = torch.randint(0x3A00, 0x3D80, (V,), dtype=torch.int32, device=dev(), generator=g).to(torch.int16)
    scale = scale.view(torch.bfloat16)
    x = torch.randn((M, H), device=dev(), generator=g).to(torch.bfloat16)
    log(f"lm_head full vocabulary V={V} H={H} M={M}")
    out = exl3.lm_head_int8(x, table, scale)
    torch.cuda.synchronize()
    vs = torch.cat([torch.randint(0, V, (256,), device=dev(), generator=g), torch.tensor([V - 1], device=dev())])
    got = _bits(out[:, vs].contiguous())
    rows = table[vs].cpu().numpy()
    srows = _bits(scale[vs].contiguous())
    _check(got, _bits(x), rows, srows)
    del table
    torch.cuda.empty_cache()
