"""C-ABI contract checks that need no GPU: the library loads, exports every
entry point include/csa2.h declares, sizes workspaces, and rejects bad
arguments before anything is launched (fake but aligned pointers are passed:
validation fails first, so they are never dereferenced)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

b = pytest.importorskip("sparse_long_context_csa2_amd.binding",
                        reason="libcsa2.so not built (python -m sparse_long_context_csa2_amd.build)")

A = ctypes.c_void_p(0x10000)  # aligned, never dereferenced
A2 = ctypes.c_void_p(0x20000)
MIS = ctypes.c_void_p(0x10004)  # misaligned


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"CSA2_API\s+[^;(]*?\b(csa2_\w+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_symbols()
    assert len(names) == 18, names
    lib = ctypes.CDLL(b.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(b.EXPORTS) == names
    assert "gfx950" in b.version()


def test_workspace_sizes_grow_with_problem():
    assert b._topk_ws(1, 1, 1000, 10) < b._topk_ws(1, 1, 100000, 10) < b._topk_ws(4, 1, 100000, 10)
    assert b._index_ws(b.BF16, 16, 1, 64, 128, 32768, 0) > 0
    assert b._attn_ws(b.BF16, b.BF16, 16, 1, 64, 512, 2048) > 0       # split over blocks of 128 entries
    assert b._attn_ws(b.BF16, b.BF16, 16, 1, 64, 512, 128) == 0       # one split: no partials
    assert b._compress_ws(b.F32, 1024, 512, 4, 1) >= 4100 * 512 * 4        # fp32 rows: Z through memory
    assert b._compress_ws(b.BF16, 1024, 512, 4, 1) == 512 * 512 * 2         # bf16 rows: only W^T


def _rc(fn, *args):
    return fn(*args)


def test_topk_rejects_bad_arguments_without_launching():
    ws = ctypes.c_size_t(1 << 40)
    assert _rc(b._topk, A, 1, 1, 100, None, 0, A2, None, A, ws, None) == 1          # k = 0
    assert _rc(b._topk, None, 1, 1, 100, None, 5, A2, None, A, ws, None) == 1       # scores NULL
    assert _rc(b._topk, MIS, 1, 1, 100, None, 5, A2, None, A, ws, None) == 1        # misaligned
    assert _rc(b._topk, A, 1, 1, 100, None, 5, A2, None, A, 16, None) == 3          # workspace too small
    assert "workspace" in b._last_error().decode()


def test_index_score_rejects_and_reports_unsupported():
    ws = 1 << 30
    # unknown dtype
    assert b._index(A, A, A, 4, 1, 1, 4, 64, 100, None, 1, None, 0, A2, None, A, ws, None) == 1
    # FP4 queries and keys: the matrix-core shape rule of FP4 keys, 4-byte aligned query rows, and
    # the decoded queries' room in the workspace
    assert b._index(A, A, A, b.FP4QK, 1, 1, 4, 64, 100, None, 1, None, 0, A2, None, A, ws, None) == 2
    assert b._index(MIS, A, A, b.FP4QK, 1, 1, 64, 128, 100, None, 1, None, 0, A2, None, A, ws, None) == 1
    qk = b._index_ws(b.FP4QK, 2, 3, 64, 128, 1000, 0)
    assert qk >= b._index_ws(b.FP4, 2, 3, 64, 128, 1000, 0) + 2 * 3 * 64 * 128 * 2
    # FP4 keys without a matrix-core shape (HI = 4), and with dI % 64 != 0
    assert b._index(A, A, A, 2, 1, 1, 4, 64, 100, None, 1, None, 0, A2, None, A, ws, None) == 2
    assert b._index(A, A, A, 2, 1, 1, 64, 32, 100, None, 1, None, 0, A2, None, A, ws, None) == 2
    # HI * dI beyond every kernel
    assert b._index(A, A, A, 0, 1, 1, 512, 512, 100, None, 1, None, 0, A2, None, A, ws, None) == 2
    # cand with P = 0
    assert b._index(A, A, A, 1, 1, 1, 64, 128, 100, None, 1, A, 0, A2, None, A, ws, None) == 1
    # q_pos with m = 0
    assert b._index(A, A, A, 1, 1, 1, 64, 128, 100, A, 0, None, 0, A2, None, A, ws, None) == 1


def test_attention_and_compress_validation():
    ws = 1 << 30
    # FP4 kv with fp32 queries
    assert b._attn(A, A, 0, 2, 1, 1, 16, 512, 10, A, 4, 1.0, A2, None, A, ws, None) == 1
    # FP4 kv with D % 16 != 0
    assert b._attn(A, A, 1, 2, 1, 1, 16, 40, 10, A, 4, 1.0, A2, None, A, ws, None) == 1
    # vector path beyond its LDS limit (fp32 q, k huge)
    assert b._attn(A, A, 0, 0, 1, 1, 8, 128, 10, A, 20000, 1.0, A2, None, A, ws, None) == 2
    # compress: m > 16, D % 16
    assert b._compress(A, 1, 4, 512, 17, 0, A, A, A2, A, ws, None) == 1
    assert b._compress(A, 1, 4, 40, 4, 0, A, A, A2, A, ws, None) == 1


def test_layer_mode_pointer_mismatch():
    a = b.LayerArgs()
    a.mode, a.B, a.Q, a.N, a.m, a.HI, a.dI, a.idx_dt = b.REINDEX, 1, 1, 1000, 4, 64, 128, b.BF16
    a.k, a.P, a.H, a.D, a.q_dt, a.kv_dt, a.scale = 64, 0, 64, 512, b.BF16, b.BF16, 0.04
    a.qI, a.w, a.kI, a.idx, a.q, a.kv, a.out = A, A, A, A, A, A, A2
    assert b._layer(ctypes.byref(a), A, 1 << 40, None) == 1      # REINDEX without pool slots
    a.P = 128
    assert b._layer(ctypes.byref(a), A, 1 << 40, None) == 1      # ... and without the pool pointer
    a.mode, a.P = 99, 0
    assert b._layer(ctypes.byref(a), A, 1 << 40, None) == 1      # unknown mode
    a.mode, a.idx = b.REUSE, None
    assert b._layer(ctypes.byref(a), A, 1 << 40, None) == 1      # REUSE without indices
    a.mode, a.idx = b.FULL, A
    need = b._layer_ws(ctypes.byref(a))
    assert need > 0
    assert b._layer(ctypes.byref(a), A, need - 256, None) == 3   # workspace one block short
    a.score_fmt = 7
    assert b._layer(ctypes.byref(a), A, 1 << 40, None) == 1      # unknown score format
    a.score_fmt, a.idx_dt, a.qI = b.SCORE_FMTS["bf16"], b.FP4QK, MIS
    assert b._layer(ctypes.byref(a), A, 1 << 40, None) == 1      # FP4 query rows misaligned
    a.qI = A
    assert b._layer_ws(ctypes.byref(a)) >= need + 64 * 128 * 2  # room for the decoded queries


def test_swa_merge_and_quantize_validation():
    ws = 1 << 30
    assert b._swa_ws(b.BF16, b.BF16, 2, 1, 64, 512, 128) >= 2 * 64 * 512 * 2   # the window branch's own output
    assert b._swa_ws(b.BF16, b.BF16, 2, 1, 64, 512, 0) == 0
    # csa2_swa_attn(q, swa_kv, q_dt, kv_dt, B, Q, H, D, T, q_pos, W, scale, csa_out, csa_lse, out, lse, ws, bytes, s)
    assert b._swa(A, A, b.BF16, b.BF16, 1, 1, 64, 512, 100, A, 0, 0.1, None, None, A2, None, A, ws, None) == 1  # W = 0
    assert b._swa(A, A, b.BF16, b.BF16, 1, 1, 64, 512, 100, A, 128, 0.1, A, None, A2, None, A, ws, None) == 1  # lse missing
    assert b._swa(A, A, b.BF16, b.BF16, 1, 1, 64, 512, 100, None, 128, 0.1, None, None, A2, None, A, ws, None) == 1
    assert b._swa(MIS, A, b.BF16, b.BF16, 1, 1, 64, 512, 100, A, 128, 0.1, None, None, A2, None, A, ws, None) == 1
    assert b._swa(A, A, b.BF16, b.FP4, 1, 1, 64, 40, 100, A, 128, 0.1, None, None, A2, None, A, ws, None) == 1
    assert b._swa(A, A, b.BF16, b.BF16, 1, 1, 64, 512, 100, A, 128, 0.1, None, None, A2, None, A, 16, None) == 3
    # csa2_merge_attn(o_a, lse_a, o_b, lse_b, dt, R, D, out, lse, s)
    assert b._merge(A, A, A, A, b.BF16, 10, 12, A2, None, None) == 1       # D % 8
    assert b._merge(A, A, A, A, b.BF16, 0, 64, A2, None, None) == 1        # R = 0
    assert b._merge(A, A, A, A, b.FP4, 10, 64, A2, None, None) == 1        # not a plain dtype
    assert b._merge(A, None, A, A, b.BF16, 10, 64, A2, None, None) == 1    # lse_a NULL
    # csa2_quantize_fp4(x, dt, n, D, cache, dst_row, s)
    assert b._quant(A, b.BF16, 10, 24, A2, None, None) == 1                # D % 16
    assert b._quant(A, b.BF16, 0, 64, A2, None, None) == 1                 # n = 0
    assert b._quant(A, b.FP4, 10, 64, A2, None, None) == 1                 # FP4 input
    assert b._quant(None, b.BF16, 10, 64, A2, None, None) == 1             # x NULL
    assert b._quant(A, b.BF16, 10, 64, None, None, None) == 1              # cache NULL
    assert b._quant(A, b.BF16, 10, 64, A2, MIS, None) == 1                 # dst_row misaligned
    assert "aligned" in b._last_error().decode()


def test_query_rows_beyond_the_grid_limit_are_rejected_before_launch():
    """B * Q indexes a launch's second grid dimension: more than 65535 query
    rows are refused with EUNSUPPORTED by every entry point that takes them."""
    ws = 1 << 40
    assert b._index(A, A, A, 1, 256, 257, 64, 128, 100, None, 1, None, 0, A2, None, A, ws, None) == 2
    assert "65535" in b._last_error().decode()
    assert b._topk(A, 65536, 1, 100, None, 5, A2, None, A, ws, None) == 2
    assert b._attn(A, A, 1, 1, 1, 70000, 64, 512, 10, A, 2048, 1.0, A2, None, A, ws, None) == 2
    assert b._swa(A, A, b.BF16, b.BF16, 300, 300, 64, 512, 100, A, 128, 0.1, None, None, A2, None, A, ws,
                  None) == 2
    a = b.LayerArgs()
    a.mode, a.B, a.Q, a.N, a.m, a.HI, a.dI, a.idx_dt = b.FULL, 65536, 1, 1000, 4, 64, 128, b.BF16
    a.k, a.P, a.H, a.D, a.q_dt, a.kv_dt, a.scale = 64, 0, 64, 512, b.BF16, b.BF16, 0.04
    a.qI, a.w, a.kI, a.idx, a.q, a.kv, a.out = A, A, A, A, A, A, A2
    assert b._layer(ctypes.byref(a), A, ws, None) == 2
    assert b._layer_ws(ctypes.byref(a)) == 0
    a.B = 65535
    assert b._layer(ctypes.byref(a), A, 0, None) == 3  # within the limit: only the workspace is short


def test_workspace_size_alias_and_format_alias():
    a = b.LayerArgs()
    a.mode, a.B, a.Q, a.N, a.m, a.HI, a.dI, a.idx_dt = b.FULL, 16, 1, 32768, 4, 64, 128, b.BF16
    a.k, a.P, a.H, a.D, a.q_dt, a.kv_dt, a.scale = 2048, 0, 64, 512, b.BF16, b.BF16, 0.04
    assert b._ws_alias(ctypes.byref(a)) == b._layer_ws(ctypes.byref(a)) > 0
    text = open(HEADER).read()
    assert "CSA2_FP4E2M1_S16E4M3 = 2" in text and "CSA2_FP4 = 2" in text


def test_noalloc_layer_rejects_layers_beyond_its_scratch_before_launch():
    """csa2_layer_noalloc refuses, before touching the device, a layer whose
    workspace exceeds its fixed 64 MiB scratch, and validates like csa2_layer."""
    a = b.LayerArgs()
    a.mode, a.B, a.Q, a.N, a.m, a.HI, a.dI, a.idx_dt = b.FULL, 16, 1, 1 << 20, 1, 64, 128, b.BF16
    a.k, a.P, a.H, a.D, a.q_dt, a.kv_dt, a.scale = 2048, 16384, 64, 512, b.BF16, b.FP4, 0.04
    a.qI, a.w, a.kI, a.idx, a.pool, a.q, a.kv, a.out = A, A, A, A, A, A, A, A2
    assert b._layer_ws(ctypes.byref(a)) > b.NOALLOC_SCRATCH_BYTES
    assert b._layer_noalloc(ctypes.byref(a), None) == 2
    assert "scratch" in b._last_error().decode()
    a.idx = None
    assert b._layer_noalloc(ctypes.byref(a), None) == 1   # validation first, as csa2_layer
