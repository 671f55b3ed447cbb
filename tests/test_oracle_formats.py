"""Pins for the oracle's FP4 / E4M3 decoding (format of the FP4 main KV on
"Recall之王 祭出Reuse", section "把KV Cache压到极致的几把杀手锏")."""
import math

import numpy as np
import torch

import oracle
from oracle_helpers import decode_fp4_independent, e2m1_table, e4m3_table
from sparse_long_context_csa2_amd import synth


def test_e4m3_every_byte_matches_torch_float8():
    ref = e4m3_table()
    for b in range(256):
        v = oracle.e4m3(b)
        if math.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b] and math.copysign(1, v) == math.copysign(1, ref[b]), (b, v, ref[b])


def test_e2m1_every_code_matches_ocp_table():
    ref = e2m1_table()
    for c in range(16):
        v = oracle.e2m1(c)
        assert v == ref[c] and math.copysign(1, v) == math.copysign(1, ref[c]), (c, v, ref[c])


def test_fp4_row_byte_layout_worked_example():
    # D = 32: 16 code bytes then 2 scale bytes.  Byte 0 = 0x21: channel 0 is
    # the low nibble (code 1 = 0.5), channel 1 the high nibble (code 2 = 1.0).
    # Byte 7 = 0xF7: channel 14 = code 7 (6.0), channel 15 = code 15 (-6.0).
    # Byte 8 = 0x9B: channel 16 = code 11 (-1.5), channel 17 = code 9 (-0.5).
    # Scale 0 = 0x38 (1.0) covers channels 0..15; scale 1 = 0x44 (2^1 * 1.5 = 3.0)
    # covers channels 16..31.
    row = np.zeros(18, dtype=np.uint8)
    row[0], row[7], row[8] = 0x21, 0xF7, 0x9B
    row[16], row[17] = 0x38, 0x44
    got = oracle.decode_rows(row[None, :], 32)[0]
    want = np.zeros(32)
    want[0], want[1], want[14], want[15] = 0.5, 1.0, 6.0, -6.0
    want[16], want[17] = -1.5 * 3.0, -0.5 * 3.0
    assert np.array_equal(got, want)


def test_fp4_rows_match_independent_table_decode():
    rng = np.random.default_rng(11)
    rows = synth.fp4_rows(rng, (3, 40), 64).numpy()
    got = oracle.decode_rows(rows, 64)
    want = decode_fp4_independent(rows, 64)
    assert np.array_equal(got, want)


def test_fp4_scale_nan_code_saturates_and_every_other_byte_is_e4m3():
    """Reading for scale bytes S.1111.111 (E4M3FN's NaN code, never written by
    a quantizer): the scale saturates to +-448.  Every other byte, including
    zero, negative zero, subnormals and sign-set bytes, is its E4M3 value."""
    ref = e4m3_table()
    for b in range(256):
        v = oracle.fp4_scale(b)
        if b in (0x7F, 0xFF):
            assert v == (448.0 if b == 0x7F else -448.0), (b, v)
        else:
            assert v == ref[b] and math.copysign(1, v) == math.copysign(1, ref[b]), (b, v, ref[b])
    # in a row: channel 0 = code 7 (6.0) under scale 0x7F, channel 16 = code 15 (-6.0) under 0xFF,
    # channel 32 = code 1 (0.5) under the smallest subnormal 0x01 (2^-9), channel 48 = code 2 (1.0) under 0x80
    D = 64
    row = np.zeros(D // 2 + D // 16, dtype=np.uint8)
    row[0], row[8], row[16], row[24] = 0x07, 0x0F, 0x01, 0x02
    row[32:36] = [0x7F, 0xFF, 0x01, 0x80]
    got = oracle.decode_rows(row[None, :], D)[0]
    want = np.zeros(D)
    want[0], want[16], want[32], want[48] = 6.0 * 448.0, -6.0 * -448.0, 0.5 * 2.0 ** -9, -0.0
    assert np.array_equal(got, want)
    assert math.copysign(1, got[48]) == -1.0


def test_fp4_rows_every_scale_byte_match_independent_decode():
    rng = np.random.default_rng(13)
    D = 512
    rows = rng.integers(0, 256, size=(40, D // 2 + D // 16), dtype=np.uint8)
    rows[:, D // 2:] = np.arange(40 * D // 16).reshape(40, D // 16) % 256
    assert np.array_equal(oracle.decode_rows(rows, D), decode_fp4_independent(rows, D))


def test_bf16_and_f32_rows_decode_exactly():
    rng = np.random.default_rng(5)
    x = synth.normal_bf16(rng, (4, 48))
    got = oracle.decode_rows(x, 48)
    assert np.array_equal(got, x.to(torch.float64).numpy())
    y = synth.normal_f32(rng, (2, 16))
    assert np.array_equal(oracle.decode_rows(y, 16), y.numpy().astype(np.float64))


def test_synth_fp4_scales_in_range():
    rng = np.random.default_rng(0)
    rows = synth.fp4_rows(rng, (200,), 512).numpy()
    sc = e4m3_table()[rows[:, 256:]]
    assert sc.min() >= 2.0 ** -4 and sc.max() < 2.0 ** 4
    assert rows.shape == (200, 288)
