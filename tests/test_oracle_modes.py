"""Pins for the layer modes (Full / Reindex / Reuse on the V4.1 Flash transcript
and "Recall之王 祭出Reuse"; hierarchical pool on the latter)."""
import numpy as np
import torch

import oracle
from sparse_long_context_csa2_amd import synth


def _decode(seed=0, N=300, k=20, P=60):
    spec = synth.Decode(B=2, Q=2, N=N, HI=4, dI=32, H=4, D=32, k=k, P=P, seed=seed,
                        layers=["FULL", "REINDEX", "REUSE"])
    return spec, synth.make_decode(spec)


def test_full_pool_contains_topk_and_reuse_is_attention():
    spec, d = _decode()
    L0 = d["layers"][0]
    full = oracle.layer("FULL", k=spec.k, scale=spec.scale, q=L0["q"], kv=d["kv"], qI=L0["qI"], w=L0["w"],
                        kI=d["kI"], P=spec.P)
    for b in range(2):
        for q in range(2):
            assert set(full["idx"][b, q]) <= set(full["pool"][b, q])
    L2 = d["layers"][2]
    reuse = oracle.layer("REUSE", k=spec.k, scale=spec.scale, q=L2["q"], kv=d["kv"], idx=full["idx"])
    o, l = oracle.sparse_attn(L2["q"], d["kv"], full["idx"], spec.scale)
    assert np.array_equal(reuse["out"], o) and np.array_equal(reuse["lse"], l)


def test_reindex_over_every_entry_equals_full():
    spec, d = _decode(seed=1)
    L0 = d["layers"][0]
    full = oracle.layer("FULL", k=spec.k, scale=spec.scale, q=L0["q"], kv=d["kv"], qI=L0["qI"], w=L0["w"],
                        kI=d["kI"])
    pool = torch.arange(spec.N, dtype=torch.int32).expand(2, 2, spec.N).contiguous()
    re = oracle.layer("REINDEX", k=spec.k, scale=spec.scale, q=L0["q"], kv=d["kv"], qI=L0["qI"], w=L0["w"],
                      kI=d["kI"], pool=pool)
    assert np.array_equal(re["idx"], full["idx"])
    assert np.array_equal(re["out"], full["out"])


def test_reindex_with_full_queries_reproduces_full_topk():
    spec, d = _decode(seed=2)
    L0 = d["layers"][0]
    full = oracle.layer("FULL", k=spec.k, scale=spec.scale, q=L0["q"], kv=d["kv"], qI=L0["qI"], w=L0["w"],
                        kI=d["kI"], P=spec.P)
    re = oracle.layer("REINDEX", k=spec.k, scale=spec.scale, q=L0["q"], kv=d["kv"], qI=L0["qI"], w=L0["w"],
                      kI=d["kI"], pool=full["pool"])
    assert np.array_equal(re["idx"], full["idx"])
    # own queries: the selection stays inside the pool
    L1 = d["layers"][1]
    re2 = oracle.layer("REINDEX", k=spec.k, scale=spec.scale, q=L1["q"], kv=d["kv"], qI=L1["qI"], w=L1["w"],
                       kI=d["kI"], pool=full["pool"])
    for b in range(2):
        for q in range(2):
            assert set(re2["idx"][b, q]) <= set(full["pool"][b, q])


def test_causal_row_equals_decode_over_visible_prefix():
    rng = np.random.default_rng(3)
    m, N = 4, 80
    kI = synth.normal_bf16(rng, (1, N, 16))
    qI = synth.normal_bf16(rng, (1, 2, 4, 16))
    w = synth.uniform_f32(rng, (1, 2, 4))
    pos = torch.tensor([[150, 319]])
    s = oracle.index_score(qI, w, kI, q_pos=pos, m=m)
    idx, cnt = oracle.topk(s, 10)
    for q, nvis in enumerate([37, 80]):
        sd = oracle.index_score(qI[:, q:q + 1], w[:, q:q + 1], kI[:, :nvis].contiguous())
        idd, cd = oracle.topk(sd, 10)
        assert np.array_equal(idx[0, q], idd[0, 0]) and cnt[0, q] == cd[0, 0]
