"""Pins for the oracle's BF16 score keys and FP4 indexer queries.

"读完这篇，你就搞懂 DeepSeek v4 了", the passage on V4's FP4 quantization-aware
training: the lightning indexer's q and K are FP4, while its score is quantized
only down to BF16, since top-k ranks it.  Readings (oracle/csa2_oracle.c): the
ranked key is the binary64 score rounded once to bfloat16, nearest with ties
to even, ties between keys broken by entry index; an FP4 query row has the
layout of an FP4 key row and is decoded exactly.

The rounding is checked against torch's float32 -> bfloat16 conversion (round
to nearest even) on values that float32 holds exactly, where rounding from
binary64 and from binary32 agree, and against hand-worked cases where they do
not (a value just above a bfloat16 midpoint that binary32 would round onto
it).  The keyed top-k is checked against a brute-force sort; the FP4 query path
against a hand-worked row and an independent table decode."""
import numpy as np
import torch

import oracle
from oracle_helpers import decode_fp4_independent


def _torch_bf16(x32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x32).to(torch.bfloat16).to(torch.float64).numpy()


def test_round_bf16_matches_torch_on_binary32_values():
    rng = np.random.default_rng(3)
    bits = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    # plus every float32 a few ulps around bfloat16 midpoints and binade edges
    base = rng.integers(0, 2 ** 16, size=4000, dtype=np.uint32) << 16
    near = (base[:, None] + np.array([0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x10000 - 0x8000], dtype=np.uint32)[None, :])
    y = near.ravel().view(np.float32)
    y = y[np.isfinite(y)]
    for v in (x, y):
        assert np.array_equal(oracle.round_bf16(v.astype(np.float64)), _torch_bf16(v), equal_nan=True)


def test_round_bf16_hand_worked():
    cases = [
        (1.0 + 2.0 ** -8, 1.0),                          # midpoint: ties to the even significand
        (1.0 + 3 * 2.0 ** -8, 1.0 + 2.0 ** -6),          # midpoint, even neighbour above
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 1.0 + 2.0 ** -7),  # above the midpoint: binary32 would round onto it
        (1.0 + 2.0 ** -8 - 2.0 ** -40, 1.0),
        (-(1.0 + 2.0 ** -8 + 2.0 ** -40), -(1.0 + 2.0 ** -7)),
        (200.49, 200.0), (200.5, 200.0), (201.5, 202.0), (200.5000001, 201.0),  # spacing 1 in [128, 256)
        (2.0 ** 127 * (2 - 2.0 ** -8), np.inf),           # rounds past the largest finite value
        (2.0 ** 127 * (2 - 2.0 ** -8) * (1 - 2.0 ** -40), 2.0 ** 127 * (2 - 2.0 ** -7)),
        (-1e300, -np.inf),
        (1.5 * 2.0 ** -133, 2.0 ** -132),                 # subnormal spacing 2^-133, tie to even
        (2.0 ** -134, 0.0),                               # half the smallest subnormal: tie to zero
        (2.0 ** -134 * (1 + 2.0 ** -30), 2.0 ** -133),
        (2.0 ** -126 * (1 + 2.0 ** -8), 2.0 ** -126),     # smallest normal binade, midpoint
        (0.0, 0.0), (np.inf, np.inf), (-np.inf, -np.inf),
    ]
    got = oracle.round_bf16(np.array([c[0] for c in cases]))
    for (x, want), g in zip(cases, got):
        assert g == want, (x, g, want)
    neg0 = oracle.round_bf16(np.array([-0.0]))[0]
    assert neg0 == 0.0 and np.signbit(neg0)
    assert np.isnan(oracle.round_bf16(np.array([np.nan]))[0])


def test_round_bf16_is_monotone_and_idempotent():
    rng = np.random.default_rng(5)
    x = np.sort(np.concatenate([rng.normal(0, 1, 20000) * 10.0 ** rng.integers(-40, 38, 20000),
                                rng.uniform(-300, 300, 20000)]))
    r = oracle.round_bf16(x)
    assert np.all(np.diff(r) >= 0)
    assert np.array_equal(oracle.round_bf16(r), r)
    assert np.array_equal(r, _torch_bf16(r.astype(np.float32)))  # every result is a bfloat16 value


def _brute_topk(s: np.ndarray, k: int, key) -> list:
    sel = [j for j in range(len(s)) if s[j] != -np.inf]
    sel.sort(key=lambda j: (-key(s[j]), j))
    return sorted(sel[:k])


def test_topk_bf16_keys_brute_force():
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, 45))
        # scores spread over a few bfloat16 spacings so that many round alike
        s32 = (rng.uniform(190, 196, n)).astype(np.float32)
        s32[rng.random(n) < 0.1] = -np.inf
        s = s32.astype(np.float64)
        idx, cnt = oracle.topk(s[None, :], k, key="bf16")
        tk = torch.from_numpy(s32).to(torch.bfloat16).to(torch.float64).numpy()
        want = _brute_topk(tk, k, lambda v: v)
        assert cnt[0] == len(want)
        assert list(idx[0, : cnt[0]]) == want and np.all(idx[0, cnt[0]:] == -1), trial


def test_topk_bf16_keys_hand_worked():
    # entry 1 has the higher binary64 score but rounds to the same bfloat16 as
    # entry 0, so the lower index wins the tie; entry 2 is a bfloat16 step above
    s = np.array([[1.0, 1.0 + 2.0 ** -9, 1.0 + 2.0 ** -7, 0.5]])
    idx64, _ = oracle.topk(s, 2)
    idx16, _ = oracle.topk(s, 2, key="bf16")
    assert list(idx64[0]) == [1, 2]
    assert list(idx16[0]) == [0, 2]
    # candidate slots: the tie is broken by entry index, not by slot
    cand = np.array([[7, 3, 9, 1]], dtype=np.int32)
    idx_c, _ = oracle.topk(s, 2, cand=cand, key="bf16")
    assert list(idx_c[0]) == [3, 9]


def _fp4_row(codes: dict, scales: dict, D: int) -> np.ndarray:
    row = np.zeros(D // 2 + D // 16, dtype=np.uint8)
    for c, code in codes.items():
        row[c // 2] |= (code & 15) << (4 * (c % 2))
    for g, byte in scales.items():
        row[D // 2 + g] = byte
    return row


def test_fp4_query_hand_worked():
    D = 32
    # head 0: channel 1 (high nibble of byte 0) = 6 (code 0b0111) x scale 1.0 (0x38),
    #         channel 17 = -1.5 (0b1011) x scale 0.5 (0x30)
    # head 1: channel 1 = -6 x 1.0 -> negative dot, dropped by the ReLU
    q0 = _fp4_row({1: 0x7, 17: 0xB}, {0: 0x38, 1: 0x30}, D)
    q1 = _fp4_row({1: 0xF}, {0: 0x38}, D)
    # key: channel 1 = 1.0 (0b0010) x scale 2.0 (0x40); channel 17 = 3.0 (0b0101) x scale 0.25 (0x28)
    k0 = _fp4_row({1: 0x2, 17: 0x5}, {0: 0x40, 1: 0x28}, D)
    qI = torch.from_numpy(np.stack([q0, q1])[None, None])          # [1,1,2,row]
    kI = torch.from_numpy(k0[None, None])                          # [1,1,row]
    w = torch.tensor([[[0.5, 3.0]]], dtype=torch.float32)
    s = oracle.index_score(qI, w, kI)
    # head 0: 6*2 + (-0.75)*(0.75) = 11.4375; head 1: -12 -> 0
    assert s.shape == (1, 1, 1) and s[0, 0, 0] == 0.5 * 11.4375


def test_fp4_query_matches_independent_decode():
    rng = np.random.default_rng(21)
    B, Q, HI, dI, N = 2, 3, 8, 64, 50
    rb = dI // 2 + dI // 16
    qI = rng.integers(0, 256, size=(B, Q, HI, rb), dtype=np.uint8)
    kI = rng.integers(0, 256, size=(B, N, rb), dtype=np.uint8)
    qI[..., dI // 2:] = rng.integers(0x20, 0x48, size=(B, Q, HI, dI // 16))   # moderate scales
    kI[..., dI // 2:] = rng.integers(0x20, 0x48, size=(B, N, dI // 16))
    w = rng.uniform(0, 1, size=(B, Q, HI)).astype(np.float32)
    s = oracle.index_score(torch.from_numpy(qI), torch.from_numpy(w), torch.from_numpy(kI))
    qd = decode_fp4_independent(qI.reshape(-1, rb), dI).reshape(B, Q, HI, dI)
    kd = decode_fp4_independent(kI.reshape(-1, rb), dI).reshape(B, N, dI)
    dots = np.einsum("bqhd,bnd->bqhn", qd, kd)              # exact: few-bit operands, 64 terms
    want = np.einsum("bqh,bqhn->bqn", w.astype(np.float64), np.maximum(dots, 0.0))
    assert np.allclose(s, want, rtol=1e-12, atol=1e-12)
