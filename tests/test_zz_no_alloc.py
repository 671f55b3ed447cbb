"""csa2_layer_noalloc (the entry point for callers that cannot allocate)
against csa2_layer with a workspace, through the C ABI: the same kernels on
the library's own scratch must give the same indices, pool, counts, outputs
and lse, bit for bit.  Two calls in a row, the second smaller (the scratch
keeps the first call's contents), and a Reuse layer after them."""
import numpy as np
import pytest
import torch

from gpu_helpers import dev, host
from sparse_long_context_csa2_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_csa2_amd import binding
    return binding


def _pair(b, mode, **kw):
    ref = b.Layer(mode, **kw).run()
    got = b.Layer(mode, noalloc=True, **kw).run()
    torch.cuda.synchronize()
    for name in ("idx", "pool", "count", "out", "lse"):
        r, g = getattr(ref, name), getattr(got, name)
        if r is None:
            assert g is None
            continue
        assert torch.equal(host(r), host(g)), f"{mode}: {name} differs between csa2_layer and csa2_layer_noalloc"
    return ref


@pytest.mark.parametrize("first,second", [
    (dict(B=4, N=32768, k=2048, P=0, kv_fmt="bf16"), dict(B=2, N=5000, k=512, P=0, kv_fmt="bf16")),
    (dict(B=2, N=40000, k=2048, P=4096, kv_fmt="fp4"), dict(B=1, N=3000, k=256, P=1024, kv_fmt="fp4")),
])
def test_noalloc_matches_workspace_layer_twice(b, first, second):
    for i, cfg in enumerate((first, second)):
        spec = synth.Decode(Q=1, HI=64, dI=128, H=64, D=512, seed=30 + i, layers=["FULL", "REUSE"], **cfg)
        d = synth.make_decode(spec)
        kv, kI = dev(d["kv"]), dev(d["kI"])
        lay = d["layers"][0]
        full = _pair(b, "FULL", q=dev(lay["q"]), kv=kv, k=spec.k, scale=spec.scale, qI=dev(lay["qI"]),
                     w=dev(lay["w"]), kI=kI, P=spec.P)
        _pair(b, "REUSE", q=dev(d["layers"][1]["q"]), kv=kv, k=spec.k, scale=spec.scale, idx=full.idx)
        if spec.P:
            _pair(b, "REINDEX", q=dev(lay["q"]), kv=kv, k=spec.k // 2, scale=spec.scale, qI=dev(lay["qI"]),
                  w=dev(lay["w"]), kI=kI, pool=full.pool)
