"""Shared pieces of the GPU parity tests (no method arithmetic here)."""
import numpy as np
import torch

ATOL_BF16, RTOL_BF16 = 1e-2, 2e-2   # bf16 / FP4 attention outputs
ATOL_F32, RTOL_F32 = 1e-5, 1e-5     # fp32 configuration


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
