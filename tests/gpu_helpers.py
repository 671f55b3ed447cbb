"""Shared pieces of the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

import oracle

ATOL_BF16, RTOL_BF16 = 1e-2, 2e-2   # bf16 / FP4 attention outputs
ATOL_F32, RTOL_F32 = 1e-5, 1e-5     # fp32 configuration
# lse = m + ln l of bf16 / FP4 attention: no bf16 rounding on its path, only
# fp32 arithmetic (the logits' fp32 accumulation over D channels of exact
# products, then the fp32 sum and logarithm), so its tolerance is an fp32 one:
# rtol 1e-5 is about 170 fp32 ulps, a random-walk accumulation over 512 terms
# with a factor 7 to spare; atol covers lse near 0.
ATOL_LSE, RTOL_LSE = 1e-4, 1e-5


def dev(t):
    return None if t is None else t.to("cuda").contiguous()


def host(t):
    return t.detach().cpu()


def assert_close(gpu, ref, atol, rtol, what):
    g = host(gpu).double().numpy() if isinstance(gpu, torch.Tensor) else np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (what, g.shape, ref.shape)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(g), np.isneginf(ref)), f"{what}: -inf pattern differs"
    err = np.abs(g[fin] - ref[fin])
    lim = atol + rtol * np.abs(ref[fin])
    bad = err > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outside atol={atol} rtol={rtol}; "
                           f"worst excess {float((err - lim).max()):.3e}")


def assert_scores_within_bound(scores, err, ref):
    s = host(scores).double().numpy()
    e = host(err).double().numpy()
    assert np.array_equal(np.isneginf(s), np.isneginf(ref)), "masked entries differ"
    fin = np.isfinite(ref)
    diff = np.where(fin, np.abs(s - np.where(fin, ref, 0)), 0)
    worst = (diff / e[..., None]).max()
    assert worst <= 1.0, f"fp32 score outside its bound: max |s - ref| / E = {worst}"
    return worst


def run_group(b, d, q_pos=None):
    """Run the spec's layer list on the GPU and in the oracle; compare each layer."""
    spec = d["spec"]
    kv, kI = dev(d["kv"]), dev(d["kI"])
    g_pool = g_idx = None
    r_pool = r_idx = None
    atol, rtol = (ATOL_F32, RTOL_F32) if spec.kv_fmt == "f32" else (ATOL_BF16, RTOL_BF16)
    for li, lay in enumerate(d["layers"]):
        mode = lay["mode"]
        k = spec.layer_k(mode)
        if mode == "REUSE" and g_idx is not None:
            k = g_idx.shape[-1]  # a Reuse layer takes the previous selection as it is
        kw = dict(q=dev(lay["q"]), kv=kv, k=k, scale=spec.scale)
        rkw = dict(q=lay["q"], kv=d["kv"], k=k, scale=spec.scale)
        if mode in ("FULL", "REINDEX"):
            kw.update(qI=dev(lay["qI"]), w=dev(lay["w"]), kI=kI, q_pos=dev(q_pos), m=spec.m,
                      score_fmt=spec.score_fmt)
            rkw.update(qI=lay["qI"], w=lay["w"], kI=d["kI"], q_pos=q_pos, m=spec.m, score_key=spec.score_fmt)
        if mode == "FULL":
            kw["P"] = rkw["P"] = spec.P
        elif mode == "REINDEX":
            kw["pool"], rkw["pool"] = g_pool, r_pool
        else:
            kw["idx"], rkw["idx"] = g_idx, r_idx
        g = b.layer(mode, **kw)
        torch.cuda.synchronize()
        r = oracle.layer(mode, **rkw)
        if mode != "REUSE":
            assert np.array_equal(host(g["idx"]).numpy(), r["idx"]), f"layer {li} ({mode}): idx differs"
            assert np.array_equal(host(g["count"]).numpy(), r["count"]), f"layer {li}: count differs"
            g_idx, r_idx = g["idx"], r["idx"]
        if mode == "FULL" and spec.P > 0:
            assert np.array_equal(host(g["pool"]).numpy(), r["pool"]), f"layer {li}: pool differs"
            g_pool, r_pool = g["pool"], r["pool"]
        assert_close(g["out"], r["out"], atol, rtol, f"layer {li} ({mode}) output")
        latol, lrtol = (ATOL_F32, RTOL_F32) if spec.kv_fmt == "f32" else (ATOL_LSE, RTOL_LSE)
        assert_close(g["lse"], r["lse"], latol, lrtol, f"layer {li} ({mode}) lse")
