"""Bit-exact parity of the FP4 cache-write quantizer (through the C ABI)
against the CPU oracle ("Recall之王 祭出Reuse", section
"把KV Cache压到极致的几把杀手锏": E2M1 values, one E4M3 scale per 16 channels;
reading: smallest scale with 6 s >= max |x|, nearest code, ties to even)."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev, host
from oracle_helpers import e4m3_table
from sparse_long_context_csa2_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_csa2_amd import binding
    return binding


def _tie_rows(rng, n, D):
    """Groups holding 6 s (so the scale is s) and every code boundary
    (midpoint * s) with both signs: each rounding decision is a tie."""
    e4 = e4m3_table()
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    x = np.empty((n, D), dtype=np.float32)
    for r in range(n):
        for g in range(D // 16):
            s = e4[rng.integers(0x01, 0x7F)]
            grp = np.concatenate([[6.0], mids, -mids, [0.0]]) * s
            x[r, 16 * g: 16 * g + 16] = rng.permutation(grp)
    return x


@pytest.mark.parametrize("dt", ["f32", "bf16"])
@pytest.mark.parametrize("D", [512, 16, 144])
def test_quantize_bit_exact(b, dt, D):
    rng = np.random.default_rng(D)
    draw = synth.normal_bf16 if dt == "bf16" else synth.normal_f32
    parts = [draw(rng, (301, D), std=1.0), draw(rng, (50, D), std=1e-3), draw(rng, (50, D), std=500.0)]
    ties = torch.from_numpy(_tie_rows(rng, 40, D))
    parts.append(ties.to(torch.bfloat16) if dt == "bf16" else ties)
    z = torch.zeros(3, D, dtype=parts[0].dtype)
    z[1, ::3] = 1e-30 if dt == "f32" else 2.0 ** -120          # below every scale step
    z[2, :] = 1e6                                              # saturated
    parts.append(z)
    x = torch.cat(parts)
    if dt == "bf16":
        assert torch.equal(ties.to(torch.bfloat16).float(), ties)   # ties exact in bf16
    want = oracle.quantize_fp4(x)
    got = host(b.quantize_fp4(dev(x))).numpy()
    torch.cuda.synchronize()
    assert got.shape == want.shape
    bad = np.argwhere(got != want)
    assert len(bad) == 0, f"{len(bad)} bytes differ, first at {bad[:3].tolist()}"


def test_quantize_scatter_into_cache(b):
    rng = np.random.default_rng(5)
    n, D, rows = 200, 512, 1000
    x = synth.normal_bf16(rng, (n, D))
    dst = torch.from_numpy(rng.permutation(rows)[:n].astype(np.int64))
    cache = torch.full((rows, D // 2 + D // 16), 0xA5, dtype=torch.uint8)
    got = host(b.quantize_fp4(dev(x), cache=dev(cache), dst_row=dev(dst)))
    torch.cuda.synchronize()
    want = torch.from_numpy(oracle.quantize_fp4(x))
    assert torch.equal(got[dst], want)
    untouched = torch.ones(rows, dtype=torch.bool)
    untouched[dst] = False
    assert torch.all(got[untouched] == 0xA5)


def test_decode_time_append(b):
    """Decode-time append: every m tokens, compress the last 2m tokens (one
    entry, previous group as halo) and write the entry into each sequence's
    FP4 cache at its position; the cache bytes equal the oracle's quantizer
    applied to the compressed rows, which meet the compression tolerance."""
    rng = np.random.default_rng(9)
    B, D, m, cap = 3, 512, 4, 64
    pos = [5, 17, 40]                                   # entry index appended per sequence
    wz = synth.normal_bf16(rng, (D, D), std=1 / math.sqrt(D))
    bias = synth.normal_f32(rng, (2 * m, D), std=0.5)
    cache = torch.zeros(B * cap, D // 2 + D // 16, dtype=torch.uint8, device="cuda")
    rows = []
    for bb in range(B):
        x = synth.normal_bf16(rng, (2 * m, D))          # previous group + the new group
        e = b.compress(dev(x), n_out=1, m=m, halo=1, wz=dev(wz), bias=dev(bias))
        ref = oracle.compress(x, n_out=1, m=m, halo=1, wz=wz, bias=bias)
        g = host(e).double().numpy()
        assert np.all(np.abs(g - ref) <= 1e-2 + 2e-2 * np.abs(ref))
        rows.append(e)
    E = torch.cat(rows)                                   # [B, D] bf16 on the device
    dst = torch.tensor([bb * cap + pos[bb] for bb in range(B)], dtype=torch.int64, device="cuda")
    b.quantize_fp4(E, cache=cache, dst_row=dst)
    torch.cuda.synchronize()
    want = oracle.quantize_fp4(host(E))
    got = host(cache).numpy()
    for bb in range(B):
        assert np.array_equal(got[bb * cap + pos[bb]], want[bb])
    assert int((host(cache).sum(dim=1) != 0).sum()) <= B


def test_quantize_full_cache_sampled(b):
    """A 128K-context cache's worth of rows (16 x 32,768 x 512 bf16 in one
    launch), sampled rows checked bit-exact."""
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    n, D = 16 * 32768, 512
    x = torch.randn(n, D, generator=g, device="cuda").to(torch.bfloat16)
    cache = b.quantize_fp4(x)
    torch.cuda.synchronize()
    rs = np.random.default_rng(0).choice(n, size=512, replace=False)
    rs = np.concatenate([rs, [0, n - 1]])
    want = oracle.quantize_fp4(host(x[torch.from_numpy(rs).cuda()]))
    assert np.array_equal(host(cache[torch.from_numpy(rs).cuda()]).numpy(), want)
