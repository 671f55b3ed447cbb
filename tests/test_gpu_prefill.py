"""Prefill-chunk attention on the GPU against the oracle.

"读完这篇，你就搞懂 DeepSeek v4 了", section "注意力计算（对应步骤三）", eq. (9):
the same shared-KV attention as in decode, for a chunk of many query tokens
per sequence.  With 64 or more query tokens per sequence, bf16 rows of 512
and more than 128 entries, csa2_sparse_attn takes each query's whole entry
list in one block (64-row tiles copied global->LDS, online softmax) instead
of 128-entry splits and a merge.  Outputs within the bf16 tolerance of the
oracle; ragged k, -1 padding, out-of-range entries, a query with no entry;
and a query's result independent of the batch it is computed in."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import ATOL_BF16, ATOL_LSE, RTOL_BF16, RTOL_LSE, assert_close, dev, host
from sparse_long_context_csa2_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_csa2_amd import binding
    return binding


def _idx(rng, B, Q, N, k, pad_max):
    out = np.full((B, Q, k), -1, dtype=np.int32)
    for bb in range(B):
        for qq in range(Q):
            kk = k - int(rng.integers(0, pad_max + 1))
            out[bb, qq, :kk] = np.sort(rng.choice(N, size=kk, replace=False))
    return out


@pytest.mark.parametrize("B,Q,H,N,k,pad", [
    (1, 64, 64, 3000, 700, 30),     # ragged: 10 full tiles and one of 60, -1 padding
    (2, 64, 128, 1500, 1024, 0),    # two head groups per query, whole tiles
    (1, 80, 64, 400, 130, 2),       # just past one split: three tiles, the last of 2 rows
])
def test_prefill_attention_matches_oracle(b, B, Q, H, N, k, pad):
    rng = np.random.default_rng(N + k)
    D = 512
    kv = synth.normal_bf16(rng, (B, N, D))
    q = synth.normal_bf16(rng, (B, Q, H, D))
    idx = _idx(rng, B, Q, N, k, pad)
    idx[0, 3] = -1                            # a query with no entry
    idx[0, 5, 10] = N + 7                     # out of range: skipped like -1
    idx = torch.from_numpy(idx)
    scale = 1 / math.sqrt(D)
    out, lse = b.sparse_attn(dev(q), dev(kv), dev(idx), scale)
    torch.cuda.synchronize()
    ref_idx = idx.clone()
    ref_idx[0, 5, 10] = -1
    ro, rl = oracle.sparse_attn(q, kv, ref_idx, scale)
    assert torch.equal(host(out[0, 3]).float(), torch.zeros(H, D))
    assert torch.isneginf(host(lse[0, 3])).all()
    assert_close(out, ro, ATOL_BF16, RTOL_BF16, "prefill attention output")
    assert_close(lse, rl, ATOL_LSE, RTOL_LSE, "prefill attention lse")


def test_prefill_attention_batch_invariance(b):
    rng = np.random.default_rng(5)
    B, Q, H, D, N, k = 3, 64, 64, 512, 2000, 1500
    kv = synth.normal_bf16(rng, (B, N, D))
    q = synth.normal_bf16(rng, (B, Q, H, D))
    idx = torch.from_numpy(_idx(rng, B, Q, N, k, 0))
    out, lse = b.sparse_attn(dev(q), dev(kv), dev(idx), 0.05)
    o1, l1 = b.sparse_attn(dev(q[1:2]), dev(kv[1:2]), dev(idx[1:2]), 0.05)
    torch.cuda.synchronize()
    assert torch.equal(host(out[1]), host(o1[0])) and torch.equal(host(lse[1]), host(l1[0]))


def test_prefill_index_scores_within_bound(b):
    """The chunk indexer (64 or more query tokens per sequence, 64 heads x 128
    bf16): query tiles of 32 with a ragged last one (70 = 32 + 32 + 6), a
    ragged last key tile, causal visibility per query token."""
    from gpu_helpers import assert_scores_within_bound
    rng = np.random.default_rng(77)
    B, Q, N, HI, dI, m = 2, 70, 3000, 64, 128, 4
    T = N * m
    kI = synth.normal_bf16(rng, (B, N, dI))
    qI = synth.normal_bf16(rng, (B, Q, HI, dI))
    w = synth.uniform_f32(rng, (B, Q, HI))
    q_pos = torch.arange(T - 300 - Q, T - 300, dtype=torch.int64).view(1, Q).repeat(B, 1)
    q_pos[1] -= 2000                                   # the second sequence further back
    ref = oracle.index_score(qI, w, kI, q_pos=q_pos, m=m)
    s, e = b.index_score(dev(qI), dev(w), dev(kI), q_pos=dev(q_pos), m=m)
    torch.cuda.synchronize()
    worst = assert_scores_within_bound(s, e, ref)
    print(f"prefill indexer: max |s - ref| / E = {worst:.3e}")


@pytest.mark.parametrize("score_fmt", ["f64", "bf16"])
def test_prefill_full_layer_with_pool(b, score_fmt):
    """A Full layer (with a pool) over a causal chunk of 96 query tokens per
    sequence: idx, pool and count bit-exact, outputs within tolerance."""
    from gpu_helpers import run_group
    spec = synth.Decode(B=2, Q=96, N=2500, HI=64, dI=128, H=64, D=512, k=400, P=800, seed=91,
                        layers=["FULL", "REINDEX", "REUSE"], score_fmt=score_fmt)
    d = synth.make_decode(spec)
    T = spec.N * spec.m
    q_pos = torch.arange(T - spec.Q, T, dtype=torch.int64).view(1, spec.Q).repeat(spec.B, 1)
    q_pos[0] -= 777
    run_group(b, d, q_pos=q_pos)


@pytest.mark.parametrize("idx_dtype,kv_fmt,score_fmt", [
    ("bf16", "bf16", "f64"),
    ("bf16", "bf16", "bf16"),
    ("f32", "f32", "f64"),
])
def test_many_queries_band_rescoring(b, idx_dtype, kv_fmt, score_fmt):
    """320 query rows (2 x 160 causal tokens): the band rescoring's grid has
    one block per query, which walks its band in rounds.  A Full layer with a
    pool (two targets' bands) and a Reindex layer over that pool (slots mapped
    through the candidates): idx, pool and count bit-exact, outputs within
    tolerance."""
    from gpu_helpers import run_group
    spec = synth.Decode(B=2, Q=160, N=1500, HI=64, dI=128, H=16, D=128, k=150, P=400, seed=93,
                        idx_dtype=idx_dtype, kv_fmt=kv_fmt, layers=["FULL", "REINDEX"], score_fmt=score_fmt)
    d = synth.make_decode(spec)
    T = spec.N * spec.m
    q_pos = torch.arange(T - spec.Q, T, dtype=torch.int64).view(1, spec.Q).repeat(spec.B, 1)
    q_pos[1] -= 333
    run_group(b, d, q_pos=q_pos)
