"""Layer-mode parity (FULL / REINDEX / REUSE) of csa2_layer against the oracle:
index sets and pools bit-exact, outputs within tolerance."""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import dev, host, run_group
from sparse_long_context_csa2_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_csa2_amd import binding
    return binding


def test_tiny_full_layer(b):
    run_group(b, synth.make_decode(synth.tiny_full(seed=0)))


def test_decode_bf16_reduced(b):
    run_group(b, synth.make_decode(synth.decode_128k(seed=1, B=2, N=5000)))


def test_decode_fp4_full_plus_five_reuse_reduced(b):
    run_group(b, synth.make_decode(synth.decode_128k_fp4_group(seed=2, B=2, N=4100)))


def test_hierarchical_full_pool_plus_reindex_reduced(b):
    spec = synth.Decode(B=2, Q=1, N=20000, HI=64, dI=128, H=64, D=512, k=512, kv_fmt="fp4", P=2048, seed=3,
                        layers=["FULL", "REINDEX", "REINDEX", "REUSE"])
    run_group(b, synth.make_decode(spec))


def test_v41_decoder_schedule_reduced(b):
    """V4.1's decoder schedule (1 Full + 3 Reuse, then 4 x (1 Reindex + 3 Reuse),
    one persistent pool, m = 1, Reindex top-k below the Full layer's), scaled down."""
    run_group(b, synth.make_decode(synth.v41_decoder_schedule(seed=4, B=2, N=9000, P=2048, k=512, k_reindex=128)))


def test_v41_encoder_schedule_reduced(b):
    """V4.1's encoder schedule (3 x (1 Full + 5 Reuse) at m = 2), scaled down."""
    run_group(b, synth.make_decode(synth.v41_encoder_schedule(seed=5, B=2, N=4500, k=512)))


def test_causal_queries_reduced(b):
    spec = synth.Decode(B=1, Q=6, N=3000, HI=64, dI=128, H=16, D=128, k=256, P=1024, seed=5,
                        layers=["FULL", "REINDEX", "REUSE"])
    pos = torch.tensor([[0, 3, 4, 1500, 11000, 11999]], dtype=torch.int64)
    run_group(b, synth.make_decode(spec), q_pos=pos)


def test_small_shapes_and_edge_k(b):
    # k above the number of entries; H = 16 heads; tiny N; vector attention for an odd D
    for spec in [synth.Decode(B=1, Q=1, N=40, HI=16, dI=64, H=16, D=64, k=64, seed=6),
                 synth.Decode(B=3, Q=1, N=1, HI=16, dI=32, H=16, D=128, k=4, seed=7),
                 synth.Decode(B=1, Q=2, N=300, HI=4, dI=64, H=8, D=128, k=50, idx_dtype="f32", kv_fmt="f32",
                              P=100, seed=8, layers=["FULL", "REINDEX", "REUSE"])]:
        run_group(b, synth.make_decode(spec))


def test_rerun_is_bitwise_deterministic(b):
    d = synth.make_decode(synth.decode_128k(seed=9, B=2, N=3000))
    lay = d["layers"][0]
    kw = dict(q=dev(lay["q"]), kv=dev(d["kv"]), k=256, scale=d["spec"].scale, qI=dev(lay["qI"]), w=dev(lay["w"]),
              kI=dev(d["kI"]))
    g1 = b.layer("FULL", **kw)
    g2 = b.layer("FULL", **kw)
    torch.cuda.synchronize()
    for key in ("idx", "out", "lse"):
        assert torch.equal(g1[key], g2[key]), key


@pytest.mark.parametrize("HI,dI,idx_dtype", [
    (8, 256, "f32"),     # 1 KiB indexer rows: the one-wave-per-entry rescoring kernel
    (16, 40, "bf16"),    # 5 vectors per row
    (100, 24, "f32"),    # more heads than lanes: head sums carried across two passes
    (128, 64, "bf16"),   # matrix-core indexer with two head passes
])
def test_certified_rescoring_row_shapes(b, HI, dI, idx_dtype):
    spec = synth.Decode(B=1, Q=2, N=3000, HI=HI, dI=dI, H=16, D=128, k=256, idx_dtype=idx_dtype, seed=HI + dI,
                        layers=["FULL"])
    run_group(b, synth.make_decode(spec))


@pytest.mark.parametrize("N,distinct,k", [
    (6000, 3, 512),    # tie groups of 2,000 entries: a band of thousands, ranked from LDS
    (9000, 2, 1024),   # a band of 4,500 entries: more than the attention prologue stages in LDS
    (5000, 40, 700),   # bands of a few hundred entries
])
def test_full_layer_tied_index_keys(b, N, distinct, k):
    """Repeated indexer keys make runs of equal scores; the lower slot wins each tie."""
    spec = synth.Decode(B=2, Q=1, N=N, HI=64, dI=128, H=64, D=512, k=k, seed=N + distinct, layers=["FULL"])
    d = synth.make_decode(spec)
    reps = torch.arange(N) % distinct
    d["kI"] = d["kI"][:, reps].contiguous()
    run_group(b, d)


@pytest.mark.parametrize("N", [20000, 70001])
def test_fp4_indexer_keys_full_pool_reindex(b, N):
    """FP4 indexer keys (bf16 queries): Full layer with a pool, Reindex layers in
    the pool, Reuse; index sets bit-exact.  70,001 entries take the selection
    path for more than 32,768 slots."""
    spec = synth.Decode(B=2, Q=1, N=N, HI=64, dI=128, H=64, D=512, k=512, kv_fmt="fp4", P=2048, seed=13,
                        idx_dtype="fp4", layers=["FULL", "REINDEX", "REUSE"])
    run_group(b, synth.make_decode(spec))


@pytest.mark.parametrize("score_fmt", ["f64", "bf16"])
def test_selection_paths_agree_across_batch_sizes(b, score_fmt):
    """Up to 16 queries the band's binary64 rescoring runs inside the one-block
    selection kernel (16 replicas of each query's block, 32 with at most 8
    queries, 64 with at most 4); with more queries a separate rescoring kernel
    does it.  17 queries and their first 16, 8 and 4 alone must select the
    same sets and pools, and give the same outputs bit for bit."""
    spec = synth.Decode(B=17, Q=1, N=6000, HI=64, dI=128, H=64, D=512, k=512, P=1024, seed=21, layers=["FULL"],
                        score_fmt=score_fmt)
    d = synth.make_decode(spec)
    lay = d["layers"][0]

    def run(nb):
        return b.layer("FULL", q=dev(lay["q"][:nb]), kv=dev(d["kv"][:nb]), k=spec.k, scale=spec.scale,
                       qI=dev(lay["qI"][:nb]), w=dev(lay["w"][:nb]), kI=dev(d["kI"][:nb]), m=spec.m, P=spec.P,
                       score_fmt=score_fmt)

    g17 = run(17)
    for nb in (16, 8, 4):
        g = run(nb)
        torch.cuda.synchronize()
        for key in ("idx", "count", "pool", "out", "lse"):
            assert torch.equal(host(g17[key])[:nb], host(g[key])), (nb, key)
    r = oracle.layer("FULL", q=lay["q"], kv=d["kv"], k=spec.k, scale=spec.scale, qI=lay["qI"], w=lay["w"], kI=d["kI"],
                     m=spec.m, P=spec.P, score_key=score_fmt)
    assert np.array_equal(host(g17["idx"]).numpy(), r["idx"])
    assert np.array_equal(host(g17["pool"]).numpy(), r["pool"])
