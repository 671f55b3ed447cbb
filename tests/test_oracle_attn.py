"""Pins for the oracle's shared-KV sparse attention ("读完这篇，你就搞懂 DeepSeek v4 了",
section "注意力计算（对应步骤三）", eq. 9: softmax attention of every query head
over the selected entries, one matrix C used as keys and values)."""
import math

import numpy as np
import torch

import oracle
from oracle_helpers import decode_fp4_independent
from sparse_long_context_csa2_amd import synth


def test_all_entries_equals_dense_sdpa():
    rng = np.random.default_rng(0)
    B, Q, H, D, N = 2, 2, 4, 32, 50
    kv = synth.normal_bf16(rng, (B, N, D))
    q = synth.normal_bf16(rng, (B, Q, H, D))
    idx = torch.arange(N, dtype=torch.int32).expand(B, Q, N).contiguous()
    scale = 1 / math.sqrt(D)
    out, lse = oracle.sparse_attn(q, kv, idx, scale)
    C = kv.to(torch.float64)
    for b in range(B):
        qq = q[b].to(torch.float64).transpose(0, 1)  # [H, Q, D]
        kk = C[b].expand(H, N, D)
        ref = torch.nn.functional.scaled_dot_product_attention(qq[None], kk[None], kk[None], scale=scale)[0]
        assert torch.allclose(torch.from_numpy(out[b]).transpose(0, 1), ref, rtol=1e-12, atol=1e-12)
        ref_lse = torch.logsumexp(scale * (qq @ C[b].T), dim=-1)  # [H, Q]
        assert torch.allclose(torch.from_numpy(lse[b]).T, ref_lse, rtol=1e-13, atol=1e-13)


def test_equal_rows_and_single_entry():
    D = 16
    row = np.linspace(-1, 1, D).astype(np.float32)
    kv = torch.from_numpy(np.tile(row, (1, 10, 1)))
    q = torch.randn(1, 1, 3, D, generator=torch.Generator().manual_seed(0))
    idx = torch.tensor([[[2, 5, 7, 9]]], dtype=torch.int32)
    out, lse = oracle.sparse_attn(q, kv, idx, 0.3)
    assert np.allclose(out[0, 0], np.tile(row.astype(np.float64), (3, 1)), rtol=0, atol=1e-15)
    a = 0.3 * (q[0, 0].double().numpy() @ row.astype(np.float64))
    assert np.allclose(lse[0, 0], a + math.log(4), rtol=1e-15, atol=1e-14)
    # one entry: the output is that row exactly, lse is its logit
    kv2 = torch.randn(1, 10, D, generator=torch.Generator().manual_seed(1))
    out, lse = oracle.sparse_attn(q, kv2, torch.tensor([[[6, -1, -1]]], dtype=torch.int32), 0.5)
    assert np.array_equal(out[0, 0], np.tile(kv2[0, 6].double().numpy(), (3, 1)))
    assert np.allclose(lse[0, 0], 0.5 * (q[0, 0].double().numpy() @ kv2[0, 6].double().numpy()), rtol=1e-15)


def test_padding_skipped_order_free_and_empty():
    rng = np.random.default_rng(2)
    kv = synth.normal_bf16(rng, (1, 30, 32))
    q = synth.normal_bf16(rng, (1, 1, 2, 32))
    idx = torch.tensor([[[3, 8, 11, 29]]], dtype=torch.int32)
    o1, l1 = oracle.sparse_attn(q, kv, idx, 0.2)
    o2, l2 = oracle.sparse_attn(q, kv, torch.tensor([[[3, -1, 8, 11, -1, 29]]], dtype=torch.int32), 0.2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    o3, l3 = oracle.sparse_attn(q, kv, torch.tensor([[[29, 11, 3, 8]]], dtype=torch.int32), 0.2)
    assert np.allclose(o1, o3, rtol=1e-14, atol=1e-15) and np.allclose(l1, l3, rtol=1e-15)
    o4, l4 = oracle.sparse_attn(q, kv, torch.full((1, 1, 4), -1, dtype=torch.int32), 0.2)
    assert np.array_equal(o4, np.zeros_like(o4)) and np.all(np.isneginf(l4))


def test_fp4_kv_equals_attention_over_decoded_values():
    rng = np.random.default_rng(3)
    D = 64
    rows = synth.fp4_rows(rng, (1, 20), D)
    dec = decode_fp4_independent(rows.numpy(), D).astype(np.float32)  # exact in fp32
    q = synth.normal_bf16(rng, (1, 2, 3, D))
    idx = torch.tensor([[[0, 5, 6, 19], [1, 2, 3, -1]]], dtype=torch.int32)
    o1, l1 = oracle.sparse_attn(q, rows, idx, 0.125)
    o2, l2 = oracle.sparse_attn(q, torch.from_numpy(dec), idx, 0.125)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
