"""Pins for the oracle's token compression (the CSA compression that
"读完这篇，你就搞懂 DeepSeek v4 了" defines by contrast in its HCA "压缩机制"
paragraphs, eqs. 10 and 11: two consecutive groups of m tokens concatenated,
per-channel softmax weights over projection Z plus learnable bias B)."""
import math

import numpy as np
import torch

import oracle
from sparse_long_context_csa2_amd import synth


def test_zero_projection_is_window_mean():
    rng = np.random.default_rng(0)
    m, D, n = 4, 16, 6
    x = synth.normal_bf16(rng, (n * m, D))
    out = oracle.compress(x, n, m, 0, torch.zeros(D, D, dtype=torch.bfloat16), torch.zeros(2 * m, D))
    X = x.to(torch.float64).numpy()
    assert np.allclose(out[0], X[0:m].mean(0), rtol=1e-15, atol=1e-15)  # entry 0: own group only
    for i in range(1, n):
        assert np.allclose(out[i], X[(i - 1) * m:(i + 1) * m].mean(0), rtol=1e-15, atol=1e-15)


def test_projection_orientation_closed_form():
    # m = 1, D = 2, entry 1 pools tokens 0 and 1 (x0 = e0, x1 = e1), bias 0.
    # Channel c's logit for token t is x_t . W[:, c] = W[t][c], so
    #   out[1][0] = x0[0] p0 + x1[0] p1 = e^W00 / (e^W00 + e^W10)
    #   out[1][1] = x0[1] p0 + x1[1] p1 = e^W11 / (e^W01 + e^W11)
    W = torch.tensor([[math.log(3), math.log(5)], [0.0, math.log(7)]], dtype=torch.float32)
    x = torch.eye(2, dtype=torch.float32)
    out = oracle.compress(x, 2, 1, 0, W, torch.zeros(2, 2))
    w = W.double().numpy()
    assert math.isclose(out[1, 0], math.exp(w[0, 0]) / (math.exp(w[0, 0]) + math.exp(w[1, 0])), rel_tol=1e-15)
    assert math.isclose(out[1, 1], math.exp(w[1, 1]) / (math.exp(w[0, 1]) + math.exp(w[1, 1])), rel_tol=1e-15)
    assert abs(out[1, 0] - 0.75) < 1e-6 and abs(out[1, 1] - 7 / 12) < 1e-6


def test_bias_row_selects_window_position():
    rng = np.random.default_rng(1)
    m, D, n = 2, 8, 5
    x = synth.normal_f32(rng, (n * m, D))
    for r in range(2 * m):
        bias = torch.zeros(2 * m, D)
        bias[r] = 60.0  # dominant logit at window position r
        out = oracle.compress(x, n, m, 0, torch.zeros(D, D), bias)
        for i in range(n):
            t = (i - 1) * m + r
            if t >= 0:
                assert np.allclose(out[i], x[t].double().numpy(), rtol=0, atol=1e-20)
        if r < m:  # entry 0 has no previous group: mean of its own group
            assert np.allclose(out[0], x[0:m].double().numpy().mean(0), rtol=1e-15)


def test_constant_channel_and_chunked_equals_whole():
    rng = np.random.default_rng(2)
    m, D, n = 4, 32, 12
    x = synth.normal_bf16(rng, (n * m, D))
    wz = synth.normal_bf16(rng, (D, D), std=0.02)
    bias = synth.normal_f32(rng, (2 * m, D), std=0.02)
    whole = oracle.compress(x, n, m, 0, wz, bias)
    # entries 5..11 from a chunk that starts one group early (halo)
    part = oracle.compress(x[4 * m:], n - 5, m, 1, wz, bias)
    assert np.array_equal(part, whole[5:])
    # a channel that is constant over all tokens pools to that constant
    x2 = x.clone()
    x2[:, 3] = 1.25
    out = oracle.compress(x2, n, m, 0, wz, bias)
    assert np.allclose(out[:, 3], 1.25, rtol=1e-15)
