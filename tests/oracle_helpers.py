"""Independent helpers for the oracle pins (no oracle arithmetic is reused)."""
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def e2m1_table():
    vals = {}
    with open(os.path.join(GOLDEN, "e2m1_ocp_mx_v1.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            vals[int(c)] = float(v)
    return np.array([vals[c] for c in range(16)], dtype=np.float64)


def e4m3_table():
    """E4M3FN byte -> value via torch's float8_e4m3fn conversion (a library routine)."""
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def decode_fp4_independent(rows: np.ndarray, D: int) -> np.ndarray:
    """FP4 rows -> float64 with table lookups (golden E2M1 table, torch E4M3)."""
    rows = np.asarray(rows, dtype=np.uint8)
    codes = rows[..., : D // 2]
    scales = rows[..., D // 2: D // 2 + D // 16]
    nib = np.empty(codes.shape[:-1] + (D,), dtype=np.uint8)
    nib[..., 0::2] = codes & 15
    nib[..., 1::2] = codes >> 4
    val = e2m1_table()[nib]
    table = e4m3_table()
    table[0x7F], table[0xFF] = 448.0, -448.0  # the NaN code as a scale saturates (reading)
    sc = np.repeat(table[scales], 16, axis=-1)
    return val * sc


def bf16(a):
    return torch.as_tensor(np.asarray(a, dtype=np.float32)).to(torch.bfloat16)
