"""Pins for the oracle's lightning-indexer score ("读完这篇，你就搞懂 DeepSeek v4 了",
section "闪电索引机制（对应步骤二）", eq. 8: per-head ReLU dot products, weighted
per head and summed)."""
from fractions import Fraction

import numpy as np
import torch

import oracle
from sparse_long_context_csa2_amd import synth


def _t(a):
    return torch.tensor(np.asarray(a, dtype=np.float32))


def test_worked_example_two_heads():
    # Keys are the unit vectors, so head h's dot with entry j is q_h[j]:
    #   head 0 dots [1, -2, 3, 0.5]  -> ReLU [1, 0, 3, 0.5]
    #   head 1 dots [-1, 4, 2, -3]   -> ReLU [0, 4, 2, 0]
    # w = [0.5, 0.25]: s = 0.5*[1,0,3,.5] + 0.25*[0,4,2,0] = [0.5, 1.0, 2.0, 0.25]
    qI = _t([[[[1, -2, 3, 0.5], [-1, 4, 2, -3]]]])
    w = _t([[[0.5, 0.25]]])
    kI = _t([np.eye(4)])
    s = oracle.index_score(qI, w, kI)
    assert s.shape == (1, 1, 4)
    assert list(s[0, 0]) == [0.5, 1.0, 2.0, 0.25]


def test_single_head_unit_weight_is_relu_of_numpy_dot():
    rng = np.random.default_rng(1)
    kI = synth.normal_bf16(rng, (2, 300, 64))
    qI = synth.normal_bf16(rng, (2, 3, 1, 64))
    w = torch.ones(2, 3, 1)
    s = oracle.index_score(qI, w, kI)
    k64 = kI.to(torch.float64).numpy()
    q64 = qI.to(torch.float64).numpy()
    for b in range(2):
        for q in range(3):
            ref = np.maximum(k64[b] @ q64[b, q, 0], 0.0)
            assert np.allclose(s[b, q], ref, rtol=1e-13, atol=1e-12)
    assert (s == 0).any() and (s > 0).any()  # both sides of the ReLU are exercised


def test_exact_rational_value_within_rounding_bound():
    rng = np.random.default_rng(2)
    HI, dI, N = 5, 24, 40
    kI = synth.normal_bf16(rng, (1, N, dI))
    qI = synth.normal_bf16(rng, (1, 1, HI, dI))
    w = synth.uniform_f32(rng, (1, 1, HI))
    s = oracle.index_score(qI, w, kI)[0, 0]
    K = kI.to(torch.float64).numpy()[0]
    Qm = qI.to(torch.float64).numpy()[0, 0]
    W = w.numpy().astype(np.float64)[0, 0]
    u = 2.0 ** -53
    for j in range(N):
        exact = Fraction(0)
        mag = 0.0
        for h in range(HI):
            d = sum(Fraction(Qm[h, i]) * Fraction(K[j, i]) for i in range(dI))
            r = d if d > 0 else Fraction(0)
            exact += Fraction(W[h]) * r
            mag += abs(W[h]) * float(sum(abs(Fraction(Qm[h, i]) * Fraction(K[j, i])) for i in range(dI)))
        bound = (dI + HI + 2) * u * mag
        assert abs(Fraction(s[j]) - exact) <= Fraction(bound), j


def test_invariants_scaling_permutation_weights():
    rng = np.random.default_rng(3)
    kI = synth.normal_bf16(rng, (1, 64, 32))
    qI = synth.normal_bf16(rng, (1, 2, 4, 32))
    w = synth.uniform_f32(rng, (1, 2, 4))
    s = oracle.index_score(qI, w, kI)
    # power-of-two scaling of the keys or the weights is exact
    assert np.array_equal(oracle.index_score(qI, w, kI * 2), 2 * s)
    assert np.array_equal(oracle.index_score(qI, w * 4, kI), 4 * s)
    # permuting entries permutes scores
    perm = rng.permutation(64)
    assert np.array_equal(oracle.index_score(qI, w, kI[:, perm]), s[:, :, perm])
    # zero weights give zero scores
    assert np.array_equal(oracle.index_score(qI, torch.zeros_like(w), kI), np.zeros_like(s))
    # negated queries flip which heads pass the ReLU; sum of both is sum_h w_h |dot_h|
    s_neg = oracle.index_score(-qI, w, kI)
    K = kI.to(torch.float64).numpy()[0]
    for q in range(2):
        Qm = qI.to(torch.float64).numpy()[0, q]
        ref = (np.abs(K @ Qm.T) * w.numpy()[0, q].astype(np.float64)).sum(1)
        assert np.allclose(s[0, q] + s_neg[0, q], ref, rtol=1e-12)


def test_causal_visibility_and_candidates():
    rng = np.random.default_rng(4)
    m, N = 4, 50
    kI = synth.normal_bf16(rng, (1, N, 16))
    qI = synth.normal_bf16(rng, (1, 3, 2, 16))
    w = synth.uniform_f32(rng, (1, 3, 2))
    full = oracle.index_score(qI, w, kI)
    pos = torch.tensor([[3, 102, 199]])  # sees floor((t+1)/4) entries: 1, 25, 50
    s = oracle.index_score(qI, w, kI, q_pos=pos, m=m)
    for q, nvis in enumerate([1, 25, 50]):
        assert np.array_equal(s[0, q, :nvis], full[0, q, :nvis])
        assert np.all(np.isneginf(s[0, q, nvis:]))
    # a query before the first complete group sees nothing
    s0 = oracle.index_score(qI[:, :1], w[:, :1], kI, q_pos=torch.tensor([[2]]), m=m)
    assert np.all(np.isneginf(s0))
    # candidate slots score their entry; -1 slots are -inf
    cand = torch.tensor([[[7, 3, -1, 49], [0, 1, 2, -1], [10, 20, 30, 40]]], dtype=torch.int32)
    sc = oracle.index_score(qI, w, kI, cand=cand)
    for q in range(3):
        for p in range(4):
            j = int(cand[0, q, p])
            if j < 0:
                assert np.isneginf(sc[0, q, p])
            else:
                assert sc[0, q, p] == full[0, q, j]


def test_bf16_values_score_like_their_f32_copies():
    rng = np.random.default_rng(6)
    kI = synth.normal_bf16(rng, (2, 40, 32))
    qI = synth.normal_bf16(rng, (2, 1, 3, 32))
    w = synth.uniform_f32(rng, (2, 1, 3))
    a = oracle.index_score(qI, w, kI)
    b = oracle.index_score(qI.float(), w, kI.float())
    assert np.array_equal(a, b)


def test_fp4_keys_score_as_their_decoded_values():
    # FP4 indexer keys: scores equal those of the independently decoded rows
    # (golden E2M1 table, torch E4M3) given as fp32, bit for bit
    from oracle_helpers import decode_fp4_independent
    rng = np.random.default_rng(21)
    B, Q, N, HI, dI = 2, 2, 90, 8, 64
    kI = synth.fp4_rows(rng, (B, N), dI)
    qI = synth.normal_bf16(rng, (B, Q, HI, dI))
    w = synth.uniform_f32(rng, (B, Q, HI))
    dec = decode_fp4_independent(kI.numpy(), dI)
    assert np.array_equal(dec.astype(np.float32).astype(np.float64), dec)
    ref = oracle.index_score(qI.float(), w, torch.from_numpy(dec.astype(np.float32)))
    got = oracle.index_score(qI, w, kI)
    assert np.array_equal(got, ref)
