"""Pins for the oracle's sliding-window (SWA) branch and its merge with the
CSA2 branch.  Video transcript on V4.1 Flash (prism.simon-ai.net), passages on
the SWA branch: a 128-token window per layer, uncompressed, never shared
across layers.  The pages give no combination rule; the reading pinned here
is one softmax over the union of both branches' entries."""
import math

import numpy as np
import torch

import oracle
from sparse_long_context_csa2_amd import synth


def test_window_idx_brute_force():
    # set definition: the W positions j with p - W < j <= p that exist (j >= 0)
    for W in (1, 3, 8, 128):
        pos = np.array([[0, 1, W - 2, W - 1, W, W + 5, 1000]], dtype=np.int64)
        idx = oracle.window_idx(pos, W)
        assert idx.shape == (1, pos.shape[1], W)
        for t, p in enumerate(pos[0]):
            want = [j for j in range(p - W + 1, p + 1) if j >= 0]
            got = idx[0, t]
            assert list(got[got >= 0]) == want
            assert np.all(got[: W - len(want)] == -1)  # padding in front, ascending after


def _attn_union_case(seed):
    rng = np.random.default_rng(seed)
    B, Q, H, D, N = 2, 3, 4, 32, 90
    kv = synth.normal_bf16(rng, (B, N, D))
    q = synth.normal_bf16(rng, (B, Q, H, D))
    perm = np.stack([np.stack([rng.permutation(N) for _ in range(Q)]) for _ in range(B)])
    ia = torch.from_numpy(np.sort(perm[..., :20], axis=-1).astype(np.int32))
    ib = torch.from_numpy(np.sort(perm[..., 20:45], axis=-1).astype(np.int32))
    return q, kv, ia, ib


def test_merge_equals_one_softmax_over_union():
    q, kv, ia, ib = _attn_union_case(1)
    scale = 1 / math.sqrt(32)
    oa, la = oracle.sparse_attn(q, kv, ia, scale)
    ob, lb = oracle.sparse_attn(q, kv, ib, scale)
    ou, lu = oracle.sparse_attn(q, kv, torch.cat([ia, ib], dim=-1), scale)
    om, lm = oracle.merge_attn(oa, la, ob, lb)
    assert np.allclose(om, ou, rtol=1e-12, atol=1e-13)
    assert np.allclose(lm, lu, rtol=1e-13, atol=1e-13)


def test_merge_empty_branch_and_symmetry():
    q, kv, ia, ib = _attn_union_case(2)
    oa, la = oracle.sparse_attn(q, kv, ia, 0.2)
    ob, lb = oracle.sparse_attn(q, kv, ib, 0.2)
    empty = torch.full_like(ib, -1)
    oe, le = oracle.sparse_attn(q, kv, empty, 0.2)
    assert np.all(le == -np.inf) and np.all(oe == 0.0)
    om, lm = oracle.merge_attn(oa, la, oe, le)
    assert np.array_equal(om, oa) and np.array_equal(lm, la)
    o0, l0 = oracle.merge_attn(oe, le, oe, le)
    assert np.all(o0 == 0.0) and np.all(l0 == -np.inf)
    o1, l1 = oracle.merge_attn(oa, la, ob, lb)
    o2, l2 = oracle.merge_attn(ob, lb, oa, la)
    assert np.allclose(o1, o2, rtol=1e-14, atol=1e-15) and np.allclose(l1, l2, rtol=1e-15, atol=0)


def test_merge_of_a_branch_with_itself():
    # two equal branches: the same output, the denominator doubled
    q, kv, ia, _ = _attn_union_case(3)
    oa, la = oracle.sparse_attn(q, kv, ia, 0.3)
    om, lm = oracle.merge_attn(oa, la, oa, la)
    assert np.allclose(om, oa, rtol=1e-14, atol=1e-15)
    assert np.allclose(lm, la + math.log(2.0), rtol=1e-14, atol=1e-14)


def test_merge_weights_by_hand():
    # one row, D = 2: branch weights e^1 and e^3 against the closed form
    oa = np.array([[1.0, -2.0]])
    ob = np.array([[4.0, 0.5]])
    om, lm = oracle.merge_attn(oa, np.array([1.0]), ob, np.array([3.0]))
    wa, wb = math.exp(1.0), math.exp(3.0)
    assert np.allclose(om[0], [(wa * 1 + wb * 4) / (wa + wb), (wa * -2 + wb * 0.5) / (wa + wb)], rtol=1e-15)
    assert math.isclose(lm[0], math.log(wa + wb), rel_tol=1e-15)


def test_swa_branch_is_attention_over_the_window():
    rng = np.random.default_rng(4)
    B, Q, H, D, T, W = 1, 3, 2, 16, 40, 8
    kv = synth.normal_bf16(rng, (B, T, D))
    q = synth.normal_bf16(rng, (B, Q, H, D))
    pos = torch.tensor([[2, 20, 39]], dtype=torch.int64)
    out, lse = oracle.swa_attn(q, kv, pos, W, 0.25)
    C = kv[0].to(torch.float64)
    for t, p in enumerate(pos[0].tolist()):
        rows = C[max(0, p - W + 1): p + 1]
        a = 0.25 * (q[0, t].to(torch.float64) @ rows.T)  # [H, n]
        ref = torch.softmax(a, dim=-1) @ rows
        assert torch.allclose(torch.from_numpy(out[0, t]), ref, rtol=1e-12, atol=1e-13)
        assert torch.allclose(torch.from_numpy(lse[0, t]), torch.logsumexp(a, dim=-1), rtol=1e-13, atol=1e-13)
