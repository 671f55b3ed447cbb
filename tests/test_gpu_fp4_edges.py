"""FP4 decode edge cases on the GPU against the oracle.

FP4 rows ("Recall之王 祭出Reuse", section "把KV Cache压到极致的几把杀手锏":
E2M1 codes, one E4M3 scale per 16 channels) whose scale bytes cover the
whole byte range: zero and negative zero, the subnormals, normals up to 448,
every sign-set byte, and the NaN code S.1111.111, which saturates to +-448
(reading; csa2.h).  Zero groups, and rows that the oracle's quantizer writes
from zero, tiny and saturated groups (scale bytes 0x00, 0x01 and 0x7E).  They
go through csa2_sparse_attn (also with bf16 queries beyond the fp16 range,
which the FP4 path prescales by a power of two), csa2_index_score with FP4
keys, and a FULL (pool) + REINDEX + REUSE group with FP4 keys and KV, whose
certified selection rescores band entries from the FP4 key rows.

Outputs are compared at the bf16 tolerance, with the absolute part scaled
down to the data when every reference value is below 1 (rows under
subnormal scales): the output is a convex combination of rows no larger
than that, so this is the same bar relative to the data's magnitude."""
import math

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import (ATOL_BF16, ATOL_LSE, RTOL_BF16, RTOL_LSE, assert_close, assert_scores_within_bound, dev, host,
                         run_group)
from sparse_long_context_csa2_amd import synth

pytestmark = pytest.mark.gpu

SUBNORMAL = list(range(0x00, 0x08)) + list(range(0x80, 0x88))           # +-0 and +-m 2^-9
SMALL = list(range(0x08, 0x40)) + list(range(0x88, 0xC0))               # 2^-6 .. < 2
LARGE = list(range(0x40, 0x7F)) + list(range(0xC0, 0xFF))               # 2 .. 448
NAN_CODE = [0x7F, 0xFF, 0x7E, 0xFE]                                     # saturating code next to +-448
ALL = list(range(256))
CLASSES = {"subnormal": SUBNORMAL, "small": SMALL, "large": LARGE, "nan_code": NAN_CODE, "all": ALL}


@pytest.fixture(scope="module")
def b():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_long_context_csa2_amd import binding
    return binding


def edge_rows(rng, lead, D, scale_bytes, zero_group_frac=0.1, quantized_rows=True):
    """FP4 rows [*lead, D/2 + D/16]: random codes, scale bytes drawn from
    scale_bytes (each byte of the list used at least once when there is room),
    some groups all-zero codes, and (optionally) rows written by the oracle's
    quantizer from zero, tiny and saturated groups."""
    n = int(np.prod(lead))
    G = D // 16
    rows = np.empty((n, D // 2 + G), dtype=np.uint8)
    rows[:, : D // 2] = rng.integers(0, 256, size=(n, D // 2), dtype=np.uint8)
    sc = np.asarray(scale_bytes, dtype=np.uint8)
    flat = rng.choice(sc, size=n * G)
    m = min(len(sc), n * G)
    flat[rng.permutation(n * G)[:m]] = sc[:m]           # every listed byte present
    rows[:, D // 2:] = flat.reshape(n, G)
    zg = rng.random((n, G)) < zero_group_frac           # groups with all codes zero
    for r, g in zip(*np.nonzero(zg)):
        rows[r, 8 * g: 8 * g + 8] = 0
    if quantized_rows and n >= 8:
        x = np.zeros((6, D), dtype=np.float32)
        x[1, ::3] = 1e-30                                 # below every scale step -> scale 0x00
        x[2, :] = 1e6                                     # saturated -> scale 0x7E, codes +-6
        x[3, :] = -1e6
        x[4, :] = 2.0 ** -10 * 6                          # smallest subnormal scale fits
        x[5, ::2] = 2.0 ** -9 * 0.25                      # tiny group: rounds to a zero code
        q = oracle.quantize_fp4(torch.from_numpy(x))
        assert {0x00, 0x7E}.issubset(set(q[:, D // 2:].ravel().tolist()))
        pos = rng.choice(n, size=6, replace=False)
        rows[pos] = q
    return torch.from_numpy(rows.reshape(*lead, D // 2 + G))


def _idx(rng, B, Q, N, k):
    out = np.empty((B, Q, k), dtype=np.int32)
    for bb in range(B):
        for qq in range(Q):
            out[bb, qq] = np.sort(rng.choice(N, size=k, replace=False))
    return torch.from_numpy(out)


def _atol_for(ref):
    big = float(np.max(np.abs(np.asarray(ref)[np.isfinite(ref)]), initial=0.0))
    return ATOL_BF16 * min(1.0, max(big, 1e-30))


@pytest.mark.parametrize("cls", list(CLASSES))
def test_sparse_attn_fp4_every_scale_byte(b, cls):
    rng = np.random.default_rng(len(CLASSES[cls]) * 7 + 1)
    B, H, D, N, k = 2, 64, 512, 2300, 640
    kv = edge_rows(rng, (B, N), D, CLASSES[cls])
    q = synth.normal_bf16(rng, (B, 1, H, D))
    idx = _idx(rng, B, 1, N, k)
    scale = 1 / math.sqrt(D)
    out, lse = b.sparse_attn(dev(q), dev(kv), dev(idx), scale, D=D)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attn(q, kv, idx, scale, D=D)
    assert np.isfinite(ro).all()
    assert_close(out, ro, _atol_for(ro), RTOL_BF16, f"attention output ({cls} scales)")
    assert_close(lse, rl, ATOL_LSE, RTOL_LSE, f"lse ({cls} scales)")


@pytest.mark.parametrize("qmax", [40000.0, 1.0e6])
def test_sparse_attn_fp4_queries_beyond_fp16_range(b, qmax):
    """bf16 queries with |q| > 32768 on FP4 KV.  The large query channels sit
    in group 0, whose scale is zero (0x00 or 0x80) in every row but a few rows
    with the smallest subnormal scale, so the logits of most rows come from
    the other, N(0,1) channels: the power-of-two prescale of the query (into
    fp16 for the matrix cores) must keep them.  It keeps them down to fp16's
    subnormal range below the largest channel, which covers queries up to
    about 2^20 times their typical channel."""
    rng = np.random.default_rng(int(qmax) % 1000 + 5)
    B, H, D, N, k = 2, 64, 512, 1500, 384
    kv = edge_rows(rng, (B, N), D, SMALL + LARGE, zero_group_frac=0.0, quantized_rows=False).numpy()
    kv[..., D // 2] = rng.choice([0x00, 0x80], size=kv.shape[:-1])      # group 0 scale: +-0
    few = rng.choice(N, size=5, replace=False)
    kv[:, few, D // 2] = 0x01                                            # ... or 2^-9 in a few rows
    kv = torch.from_numpy(kv)
    qf = synth.normal_f32(rng, (B, 1, H, D))
    big = rng.uniform(0.5, 1.0, size=(B, 1, H, 16)).astype(np.float32) * np.float32(qmax)
    qf[..., :16] = torch.from_numpy(big * np.sign(rng.standard_normal((B, 1, H, 16))).astype(np.float32))
    q = qf.to(torch.bfloat16)
    assert float(q.float().abs().max()) > 32768
    idx = _idx(rng, B, 1, N, k)
    scale = 1 / math.sqrt(D)
    out, lse = b.sparse_attn(dev(q), dev(kv), dev(idx), scale, D=D)
    torch.cuda.synchronize()
    ro, rl = oracle.sparse_attn(q, kv, idx, scale, D=D)
    assert_close(out, ro, _atol_for(ro), RTOL_BF16, "attention output (large queries)")
    assert_close(lse, rl, ATOL_LSE, RTOL_LSE, "lse (large queries)")


@pytest.mark.parametrize("cls", list(CLASSES))
def test_index_score_fp4_keys_every_scale_byte(b, cls):
    rng = np.random.default_rng(len(CLASSES[cls]) * 11 + 3)
    B, Q, N, HI, dI = 2, 1, 1800, 64, 128
    kI = edge_rows(rng, (B, N), dI, CLASSES[cls])
    qI, w = synth.normal_bf16(rng, (B, Q, HI, dI)), synth.uniform_f32(rng, (B, Q, HI))
    ref = oracle.index_score(qI, w, kI)
    s, e = b.index_score(dev(qI), dev(w), dev(kI))
    torch.cuda.synchronize()
    worst = assert_scores_within_bound(s, e, ref)
    print(f"{cls}: max |s - ref| / E = {worst:.3e}")
    # the same keys through the streaming kernel (a launch of >= 1024 tiles)
    kI2 = edge_rows(rng, (4, 70000), dI, CLASSES[cls])
    qI2, w2 = synth.normal_bf16(rng, (4, 1, HI, dI)), synth.uniform_f32(rng, (4, 1, HI))
    ref2 = oracle.index_score(qI2, w2, kI2)
    s2, e2 = b.index_score(dev(qI2), dev(w2), dev(kI2))
    torch.cuda.synchronize()
    assert_scores_within_bound(s2, e2, ref2)


@pytest.mark.parametrize("cls", ["all", "subnormal", "large"])
def test_fp4_keys_and_kv_full_pool_reindex_reuse(b, cls):
    """Certified selection on FP4 indexer keys with every scale byte of the
    class (band rescoring decodes the key rows in binary64), FP4 KV likewise;
    idx and pool bit-exact, outputs within tolerance."""
    rng = np.random.default_rng(len(CLASSES[cls]) + 17)
    spec = synth.Decode(B=2, Q=1, N=6000, HI=64, dI=128, H=64, D=512, k=512, idx_dtype="fp4", kv_fmt="fp4",
                        P=2048, seed=9, layers=["FULL", "REINDEX", "REUSE"])
    d = synth.make_decode(spec)
    d["kI"] = edge_rows(rng, (spec.B, spec.N), spec.dI, CLASSES[cls])
    d["kv"] = edge_rows(rng, (spec.B, spec.N), spec.D, CLASSES[cls])
    run_group(b, d)
