"""Pins for the oracle's FP4 quantizer for main-KV cache writes ("Recall之王
祭出Reuse", section "把KV Cache压到极致的几把杀手锏": E2M1 values with one E4M3
scale per 16 channels).  Reading (the pages give no recipe): the smallest
E4M3 scale s with 6 s >= the group's largest magnitude; each code the E2M1
value nearest to x / s, ties to the even code; a zero is +0."""
import numpy as np
import torch

import oracle
from oracle_helpers import decode_fp4_independent, e2m1_table, e4m3_table
from sparse_long_context_csa2_amd import synth


def test_hand_worked_group():
    # amax 7 -> 7/6 = 1.1667; E4M3 1.125 gives 6.75 < 7, 1.25 gives 7.5: s = 1.25 = byte 0x3A
    # (exponent field 7, mantissa 2).  x / s and the chosen codes:
    #   0.3 -> 0.24 -> 0 (code 0)        -1.1 -> -0.88 -> -1 (10)    7.0 -> 5.6 -> 6 (7)
    #   0.0 -> 0 (0)                      2.6 -> 2.08 -> 2 (4)       -5.2 -> -4.16 -> -4 (14)
    #   0.3125 = 0.25 s: tie 0 | 0.5 -> 0 (0)      0.9375 = 0.75 s: tie 0.5 | 1 -> 1 (2)
    #   1.5625 = 1.25 s: tie 1 | 1.5 -> 1 (2)      2.1875 = 1.75 s: tie 1.5 | 2 -> 2 (4)
    #   3.125 = 2.5 s: tie 2 | 3 -> 2 (4)          4.375 = 3.5 s: tie 3 | 4 -> 4 (6)
    #   6.25 = 5 s: tie 4 | 6 -> 4 (6)             -0.1 -> -0.08 -> +0 (0)
    #   0.625 = 0.5 s -> 0.5 (1)                   -7.0 -> -5.6 -> -6 (15)
    x = np.array([0.3, -1.1, 7.0, 0.0, 2.6, -5.2, 0.3125, 0.9375, 1.5625, 2.1875, 3.125, 4.375, 6.25, -0.1,
                  0.625, -7.0], dtype=np.float32)
    row = oracle.quantize_fp4(x[None])[0]
    assert list(row) == [0xA0, 0x07, 0xE4, 0x20, 0x42, 0x64, 0x06, 0xF1, 0x3A]


def test_representable_rows_round_trip():
    # rows whose every group holds a +-6 code: the scale is recovered exactly, so
    # decoding then quantizing gives the same bytes (no -0 codes: they come back as +0)
    rng = np.random.default_rng(0)
    n, D = 64, 512
    codes = rng.integers(0, 16, size=(n, D)).astype(np.uint8)
    codes[codes == 8] = 0
    codes[:, ::16] = np.where(rng.random((n, D // 16)) < 0.5, 7, 15)
    scales = rng.integers(0x01, 0x7F, size=(n, D // 16)).astype(np.uint8)  # every positive finite E4M3
    rows = np.concatenate([codes[:, 0::2] | (codes[:, 1::2] << 4), scales], axis=1)
    x = decode_fp4_independent(rows, D).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), decode_fp4_independent(rows, D))  # exact in fp32
    assert np.array_equal(oracle.quantize_fp4(x), rows)


def _check_nearest_and_minimal(x, rows, D):
    x = x.astype(np.float64).reshape(-1, D)
    rows = rows.reshape(-1, rows.shape[-1])
    e4 = e4m3_table()
    grid = e2m1_table()[:8]
    sc = e4[rows[:, D // 2:]]                                     # [n, D/16]
    amax = np.abs(x).reshape(len(x), D // 16, 16).max(-1)
    pos = e4[:0x7F]                                               # non-negative finite, increasing
    for r in range(len(x)):
        for g in range(D // 16):
            ok = np.nonzero(6 * pos >= amax[r, g])[0]
            want = pos[ok[0]] if len(ok) else 448.0
            assert sc[r, g] == want
    dec = decode_fp4_independent(rows, D)
    s = np.repeat(sc, 16, axis=-1)
    best = np.abs(np.abs(x)[..., None] - grid * s[..., None]).min(-1)
    assert np.array_equal(np.abs(np.abs(dec) - np.abs(x)), best)   # the nearest magnitude
    assert np.all((np.sign(dec) == np.sign(x)) | (dec == 0))


def test_random_rows_nearest_code_and_minimal_scale():
    rng = np.random.default_rng(1)
    for std in (1.0, 1e-3, 300.0):
        x = synth.normal_f32(rng, (8, 256), std=std).numpy()
        _check_nearest_and_minimal(x, oracle.quantize_fp4(x), 256)
        xb = synth.normal_bf16(rng, (8, 256), std=std)
        _check_nearest_and_minimal(xb.float().numpy(), oracle.quantize_fp4(xb), 256)


def test_zero_saturated_and_tiny_groups():
    x = np.zeros((1, 48), dtype=np.float32)
    x[0, 16:32] = np.linspace(-5000, 5000, 16)   # above 6 * 448: scale 448, codes saturate at +-6
    x[0, 32] = 2.0 ** -20                         # below every scale step: smallest scale, code 0
    row = oracle.quantize_fp4(x)[0]
    assert row[24] == 0x00 and np.all(row[:8] == 0)             # zero group: scale 0, codes 0
    assert row[25] == 0x7E                                      # 448
    dec = decode_fp4_independent(row[None], 48)[0]
    assert dec[16] == -6 * 448 and dec[31] == 6 * 448
    assert row[26] == 0x01 and dec[32] == 0.0                    # 2^-9 scale
