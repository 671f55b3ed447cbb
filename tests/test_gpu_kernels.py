"""Per-step parity of the HIP path (through the C ABI) against the CPU oracle:
indexer scores, exact top-k, sparse attention, compression."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (ATOL_BF16, ATOL_F32, ATOL_LSE, RTOL_BF16, RTOL_F32, RTOL_LSE, assert_close,
                         assert_scores_within_bound, dev, host)
from sparse_long_context_csa2_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_csa2_amd import binding
    return binding


# ------------------------------------------------------------------ indexer

@pytest.mark.parametrize("B,Q,N,HI,dI,dt", [
    (1, 1, 512, 4, 64, "f32"),        # tiny configuration shape (vector path)
    (2, 1, 1000, 64, 128, "bf16"),    # 128K-decode head shape, ragged N
    (1, 2, 777, 16, 64, "bf16"),
    (2, 1, 300, 32, 32, "bf16"),
    (1, 1, 513, 128, 64, "bf16"),
    (1, 1, 300, 16, 256, "bf16"),
    (1, 1, 257, 24, 40, "bf16"),      # no matrix-core variant: vector path in bf16
])
def test_index_score_within_reported_bound(b, B, Q, N, HI, dI, dt):
    rng = np.random.default_rng(N + HI)
    draw = synth.normal_bf16 if dt == "bf16" else synth.normal_f32
    kI, qI, w = draw(rng, (B, N, dI)), draw(rng, (B, Q, HI, dI)), synth.uniform_f32(rng, (B, Q, HI))
    ref = oracle.index_score(qI, w, kI)
    s, e = b.index_score(dev(qI), dev(w), dev(kI))
    torch.cuda.synchronize()
    worst = assert_scores_within_bound(s, e, ref)
    print(f"max |s - ref| / E = {worst:.3e}, E = {host(e).max().item():.3e}")


@pytest.mark.parametrize("HI,dI", [(64, 128), (128, 64), (16, 128)])
def test_index_score_streaming_path_causal_ragged(b, HI, dI):
    """Launches of at least 1024 tiles take the streaming kernel: ragged N,
    causal queries that see none, part, or all of the entries (tails inside a
    tile, inside a 64-slot step and at a tile edge)."""
    rng = np.random.default_rng(HI * dI)
    B, Q, N, m = 2, 3, 175_001, 4
    kI = synth.normal_bf16(rng, (B, N, dI))
    qI = synth.normal_bf16(rng, (B, Q, HI, dI))
    w = synth.uniform_f32(rng, (B, Q, HI))
    pos = torch.tensor([[-1, 4 * 1000 + 2, 10**7], [4 * 256 - 1, 4 * 64 * 1001 + 3, 4 * 175_000 + 1]],
                       dtype=torch.int64)
    ref = oracle.index_score(qI, w, kI, q_pos=pos, m=m)
    s, e = b.index_score(dev(qI), dev(w), dev(kI), q_pos=dev(pos), m=m)
    torch.cuda.synchronize()
    assert_scores_within_bound(s, e, ref)


def test_index_score_causal_and_candidates(b):
    rng = np.random.default_rng(7)
    N, m = 600, 4
    kI = synth.normal_bf16(rng, (1, N, 128))
    qI = synth.normal_bf16(rng, (1, 3, 64, 128))
    w = synth.uniform_f32(rng, (1, 3, 64))
    pos = torch.tensor([[2, 1001, 5000]], dtype=torch.int64)
    ref = oracle.index_score(qI, w, kI, q_pos=pos, m=m)
    s, e = b.index_score(dev(qI), dev(w), dev(kI), q_pos=dev(pos), m=m)
    torch.cuda.synchronize()
    assert_scores_within_bound(s, e, ref)
    cand = torch.tensor(rng.integers(-1, N, size=(1, 3, 300)), dtype=torch.int32)
    ref = oracle.index_score(qI, w, kI, cand=cand)
    s, e = b.index_score(dev(qI), dev(w), dev(kI), cand=dev(cand))
    torch.cuda.synchronize()
    assert_scores_within_bound(s, e, ref)


# -------------------------------------------------------------------- top-k

@pytest.mark.parametrize("n,k", [(1, 1), (31, 7), (1000, 64), (8193, 2048), (40000, 2048), (5000, 6000),
                                 (70000, 16384)])
def test_topk_exact_with_ties(b, n, k):
    rng = np.random.default_rng(n * 7 + k)
    s = (np.round(rng.standard_normal((2, 3, n)) * 8) / 8).astype(np.float32)  # heavy ties
    s[0, 1, ::5] = -np.inf
    s[1, 2, :] = -np.inf                                                        # nothing selectable
    idx, cnt = b.topk(dev(torch.from_numpy(s)), k)
    torch.cuda.synchronize()
    ri, rc = oracle.topk(s.astype(np.float64), k)
    assert np.array_equal(host(idx).numpy(), ri)
    assert np.array_equal(host(cnt).numpy(), rc)


def test_topk_all_equal_scores_band_path(b):
    n, k = 30000, 3000
    s = np.full((1, 2, n), 1.5, dtype=np.float32)
    s[0, 1, 7] = 2.0
    idx, cnt = b.topk(dev(torch.from_numpy(s)), k)
    torch.cuda.synchronize()
    ri, rc = oracle.topk(s.astype(np.float64), k)
    assert np.array_equal(host(idx).numpy(), ri) and np.array_equal(host(cnt).numpy(), rc)


def test_topk_candidates(b):
    rng = np.random.default_rng(3)
    n = 5000
    cand = np.sort(rng.choice(100000, size=(2, 1, n), replace=True), axis=-1).astype(np.int32)
    cand = np.unique(cand[0, 0])[None, None, :].repeat(2, 0)
    n = cand.shape[-1]
    cand[1, 0, n - 300:] = -1
    s = (np.round(rng.standard_normal((2, 1, n)) * 4) / 4).astype(np.float32)
    idx, cnt = b.topk(dev(torch.from_numpy(s)), 500, cand=dev(torch.from_numpy(cand)))
    torch.cuda.synchronize()
    ri, rc = oracle.topk(s.astype(np.float64), 500, cand=cand)
    assert np.array_equal(host(idx).numpy(), ri) and np.array_equal(host(cnt).numpy(), rc)


# ---------------------------------------------------------------- attention

def _idx(rng, B, Q, N, k, pad):
    out = np.full((B, Q, k), -1, dtype=np.int32)
    for bb in range(B):
        for qq in range(Q):
            kk = max(0, k - pad)
            out[bb, qq, :kk] = np.sort(rng.choice(N, size=kk, replace=False))
    return torch.from_numpy(out)


@pytest.mark.parametrize("B,Q,H,D,N,k,fmt,pad", [
    (1, 1, 8, 128, 512, 64, "f32", 0),       # tiny configuration (vector path)
    (2, 1, 64, 512, 3000, 2048, "bf16", 0),  # 128K-decode head shape, 4 splits
    (2, 1, 64, 512, 3000, 2048, "fp4", 0),
    (1, 2, 16, 128, 900, 700, "bf16", 37),   # ragged k and -1 padding
    (1, 1, 32, 256, 400, 100, "fp4", 5),
    (1, 1, 16, 64, 100, 33, "bf16", 0),
    (1, 1, 8, 96, 100, 20, "bf16", 3),       # vector path in bf16
])
def test_sparse_attn_matches_oracle(b, B, Q, H, D, N, k, fmt, pad):
    rng = np.random.default_rng(H * D + k)
    if fmt == "fp4":
        kv = synth.fp4_rows(rng, (B, N), D)
    elif fmt == "bf16":
        kv = synth.normal_bf16(rng, (B, N, D))
    else:
        kv = synth.normal_f32(rng, (B, N, D))
    q = (synth.normal_f32 if fmt == "f32" else synth.normal_bf16)(rng, (B, Q, H, D))
    idx = _idx(rng, B, Q, N, k, pad)
    scale = 1 / math.sqrt(D)
    out, lse = b.sparse_attn(dev(q), dev(kv), dev(idx), scale, D=D)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attn(q, kv, idx, scale, D=D)
    atol, rtol = (ATOL_F32, RTOL_F32) if fmt == "f32" else (ATOL_BF16, RTOL_BF16)
    assert_close(out, ro, atol, rtol, "attention output")
    assert_close(lse, rl, *((ATOL_F32, RTOL_F32) if fmt == "f32" else (ATOL_LSE, RTOL_LSE)), "lse")


@pytest.mark.parametrize("e", [24, -24])
def test_sparse_attn_split_partials_extreme_magnitudes(b, e):
    """Outputs of magnitude 2^e merged from 16 splits: the split partials are
    kept in fp16 under a power-of-two scale per quarter of the channels, which
    must follow the values up to 2^24 and down to 2^-24 without overflow or
    loss.  The KV rows are scaled by 2^e and the queries by 2^-e, so the
    logits, and the reference up to the factor 2^e, are the unscaled ones."""
    rng = np.random.default_rng(23)
    B, H, D, N, k = 1, 64, 512, 3000, 2048
    f = 2.0 ** e
    kv = (synth.normal_bf16(rng, (B, N, D)).float() * f).to(torch.bfloat16)
    q = (synth.normal_bf16(rng, (B, 1, H, D)).float() / f).to(torch.bfloat16)
    idx = _idx(rng, B, 1, N, k, 0)
    scale = 1 / math.sqrt(D)
    out, lse = b.sparse_attn(dev(q), dev(kv), dev(idx), scale, D=D)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attn(q, kv, idx, scale, D=D)
    assert_close(host(out).double() / f, np.asarray(ro) / f, ATOL_BF16, RTOL_BF16, "attention output / 2^e")
    assert_close(lse, rl, ATOL_LSE, RTOL_LSE, "lse")


def test_sparse_attn_empty_rows_and_batch_invariance(b):
    rng = np.random.default_rng(11)
    B, H, D, N, k = 16, 64, 512, 700, 1100
    kv = synth.normal_bf16(rng, (B, N, D))
    q = synth.normal_bf16(rng, (B, 1, H, D))
    idx = _idx(rng, B, 1, N, k, 400)
    idx[5] = -1  # a query with no entries
    out, lse = b.sparse_attn(dev(q), dev(kv), dev(idx), 0.05, D=D)
    o1, l1 = b.sparse_attn(dev(q[9:10]), dev(kv[9:10]), dev(idx[9:10]), 0.05, D=D)
    torch.cuda.synchronize()
    assert torch.equal(host(out[5]).float(), torch.zeros(1, H, D))
    assert torch.isneginf(host(lse[5])).all()
    assert torch.equal(host(out[9]), host(o1[0])) and torch.equal(host(lse[9]), host(l1[0]))


# -------------------------------------------------------------- compression

@pytest.mark.parametrize("n_out,D,m,halo,dt", [(40, 128, 4, 0, "bf16"), (33, 512, 4, 1, "bf16"),
                                               (17, 64, 2, 0, "f32"), (9, 48, 1, 1, "f32")])
def test_compress_matches_oracle(b, n_out, D, m, halo, dt):
    rng = np.random.default_rng(D + m)
    draw = synth.normal_bf16 if dt == "bf16" else synth.normal_f32
    rows = (n_out + halo) * m
    x = draw(rng, (rows, D))
    wz = draw(rng, (D, D), std=0.02)
    bias = synth.normal_f32(rng, (2 * m, D), std=0.02)
    out = b.compress(dev(x), n_out, m, halo, dev(wz), dev(bias))
    torch.cuda.synchronize()
    ref = oracle.compress(x, n_out, m, halo, wz, bias)
    atol, rtol = (ATOL_F32, RTOL_F32) if dt == "f32" else (ATOL_BF16, RTOL_BF16)
    assert_close(out, ref, atol, rtol, "compressed entries")


@pytest.mark.parametrize("B,Q,N,HI,dI", [(2, 1, 1000, 64, 128), (1, 2, 777, 16, 64), (1, 1, 513, 32, 256)])
def test_index_score_fp4_keys_within_reported_bound(b, B, Q, N, HI, dI):
    rng = np.random.default_rng(N + dI)
    kI = synth.fp4_rows(rng, (B, N), dI)
    qI, w = synth.normal_bf16(rng, (B, Q, HI, dI)), synth.uniform_f32(rng, (B, Q, HI))
    ref = oracle.index_score(qI, w, kI)
    s, e = b.index_score(dev(qI), dev(w), dev(kI))
    torch.cuda.synchronize()
    worst = assert_scores_within_bound(s, e, ref)
    print(f"max |s - ref| / E = {worst:.3e}")
