"""CPU oracle for the CSA2 hot path -- TEST INFRASTRUCTURE ONLY.

A thin ctypes wrapper over ``csa2_oracle.c`` (plain binary64 C, sequential
order, no fused multiply-add).  Only the tests, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package; the HIP library
and its Python binding never do, and the two share no code.

Each function states the passage of the pages it follows (page title and
section); the C file carries the full statement of each definition.

Inputs are numpy arrays or CPU torch tensors.  bf16 tensors are passed as their
raw 16-bit patterns and widened exactly inside the C code.  Floating outputs are
float64 numpy arrays.
"""
from __future__ import annotations

import ctypes
import math
import os

import numpy as np

from . import build as _build

F32, BF16, FP4 = 0, 1, 2

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        path = _build.ensure_built()
        lib = ctypes.CDLL(path)
        c_void_p, c_int, c_int64, c_double = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.ora_e2m1.argtypes, lib.ora_e2m1.restype = [ctypes.c_uint], c_double
        lib.ora_e4m3.argtypes, lib.ora_e4m3.restype = [ctypes.c_uint], c_double
        lib.ora_fp4_scale.argtypes, lib.ora_fp4_scale.restype = [ctypes.c_uint], c_double
        lib.ora_decode_row.argtypes = [c_void_p, c_int, c_int, c_void_p]
        lib.ora_compress.argtypes = [c_void_p, c_int, c_int64, c_int, c_int, c_int, c_void_p, c_void_p, c_void_p]
        lib.ora_index_score.argtypes = [c_void_p, c_void_p, c_void_p, c_int, c_int, c_int, c_int, c_int,
                                        c_int64, c_void_p, c_int, c_void_p, c_int, c_void_p]
        lib.ora_topk.argtypes = [c_void_p, c_int64, c_int64, c_void_p, c_int, c_void_p, c_void_p]
        lib.ora_sparse_attn.argtypes = [c_void_p, c_int, c_void_p, c_int, c_int, c_int, c_int, c_int, c_int64,
                                        c_void_p, c_int, c_double, c_void_p, c_void_p]
        lib.ora_window_idx.argtypes = [c_void_p, c_int64, c_int, c_void_p]
        lib.ora_quantize_fp4.argtypes = [c_void_p, c_int, c_int64, c_int, c_void_p]
        lib.ora_merge_attn.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int64, c_int, c_void_p, c_void_p]
        lib.ora_round_bf16.argtypes, lib.ora_round_bf16.restype = [c_double], c_double
        lib.ora_round_bf16_array.argtypes = [c_void_p, c_int64, c_void_p]
        for f in ("ora_decode_row", "ora_compress", "ora_index_score", "ora_topk", "ora_sparse_attn",
                  "ora_window_idx", "ora_merge_attn", "ora_quantize_fp4", "ora_round_bf16_array"):
            getattr(lib, f).restype = None
        _LIB = lib
    return _LIB


def _raw(a):
    """(contiguous numpy array, dtype code) for fp32 / bf16 / uint8 inputs."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy().view(np.uint16), BF16
            if a.dtype == torch.float32:
                return a.numpy(), F32
            if a.dtype == torch.uint8:
                return a.numpy(), FP4
            raise TypeError(f"unsupported tensor dtype {a.dtype}")
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    if a.dtype == np.uint8:
        return a, FP4
    raise TypeError(f"unsupported array dtype {a.dtype}")


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _f32(a):
    a, dt = _raw(a)
    if dt != F32:
        raise TypeError("expected float32")
    return a


def _i32(a):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(a, dtype=np.int32)


def _i64(a):
    if a is None:
        return None
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.ascontiguousarray(a, dtype=np.int64)


# ----------------------------------------------------------------- formats

def e2m1(code: int) -> float:
    """Value of a 4-bit E2M1 code (OCP MX element format)."""
    return _lib().ora_e2m1(code)


def e4m3(byte: int) -> float:
    """Value of an E4M3 ("FN") byte (OCP 8-bit floating point)."""
    return _lib().ora_e4m3(byte)


def fp4_scale(byte: int) -> float:
    """Value of an FP4 row's scale byte: its E4M3 value, except that the NaN
    code S.1111.111 saturates to +-448 (a reading: the pages give no rule)."""
    return _lib().ora_fp4_scale(byte)


def decode_rows(rows, D: int) -> np.ndarray:
    """Decode stored KV rows [..., row_bytes] (fp32, bf16 or FP4 rows) to float64 [..., D].

    FP4 rows follow "Recall之王 祭出Reuse", section "把KV Cache压到极致的几把杀手锏":
    E2M1 values with one E4M3 scale per 16 channels (byte layout in the C file).
    """
    a, dt = _raw(rows)
    width = a.shape[-1]
    lead = a.shape[:-1]
    flat = a.reshape(-1, width)
    out = np.empty((flat.shape[0], D), dtype=np.float64)
    lib = _lib()
    for r in range(flat.shape[0]):
        row = np.ascontiguousarray(flat[r])
        lib.ora_decode_row(_ptr(row), dt, D, out[r].ctypes.data_as(ctypes.c_void_p))
    return out.reshape(*lead, D)


def quantize_fp4(x) -> np.ndarray:
    """FP4 rows [..., D/2 + D/16] uint8 of fp32/bf16 rows x [..., D] (cache writes).

    "Recall之王 祭出Reuse", section "把KV Cache压到极致的几把杀手锏": E2M1 values
    with one E4M3 scale per 16 channels.  Reading (the pages give no recipe):
    the smallest E4M3 scale s with 6 s >= the group's largest magnitude, each
    code the E2M1 value nearest to x / s, ties to the even code.
    """
    a, dt = _raw(x)
    if dt == FP4:
        raise TypeError("quantize_fp4 takes fp32 or bf16 rows")
    D = a.shape[-1]
    if D % 16:
        raise ValueError("D must be a multiple of 16")
    lead = a.shape[:-1]
    flat = np.ascontiguousarray(a.reshape(-1, D))
    out = np.empty((flat.shape[0], D // 2 + D // 16), dtype=np.uint8)
    _lib().ora_quantize_fp4(_ptr(flat), dt, int(flat.shape[0]), int(D), _ptr(out))
    return out.reshape(*lead, D // 2 + D // 16)


# ------------------------------------------------------------- compression

def compress(x, n_out: int, m: int, halo: int, wz, bias) -> np.ndarray:
    """CSA token compression, float64 [n_out, D].

    "读完这篇，你就搞懂 DeepSeek v4 了", HCA "压缩机制" paragraphs (eqs. 10, 11)
    that define the CSA compression by contrast: two consecutive groups of m
    tokens concatenated, per-channel softmax weights over projection + bias.
    """
    xa, dt = _raw(x)
    wa, wdt = _raw(wz)
    if wdt != dt:
        raise TypeError("x and wz must share a dtype")
    ba = _f32(bias)
    D = xa.shape[-1]
    rows = (n_out + 1) * m if halo else n_out * m
    if xa.reshape(-1, D).shape[0] < rows:
        raise ValueError("x has too few token rows")
    if ba.shape != (2 * m, D) or wa.shape != (D, D):
        raise ValueError("bad wz / bias shape")
    out = np.empty((n_out, D), dtype=np.float64)
    _lib().ora_compress(_ptr(xa), dt, n_out, D, m, halo, _ptr(wa), _ptr(ba), _ptr(out))
    return out


# ----------------------------------------------------------------- indexer

def index_score(qI, w, kI, q_pos=None, m: int = 1, cand=None) -> np.ndarray:
    """Lightning-indexer scores, float64 [B, Q, N] (or [B, Q, P] with cand).

    "读完这篇，你就搞懂 DeepSeek v4 了", section "闪电索引机制（对应步骤二）", eq. (8):
    s(j) = sum_h w_h * ReLU(q_h . K_j); -inf for entries not visible to the
    query or empty candidate slots.
    """
    qa, dt = _raw(qI)
    ka, kdt = _raw(kI)
    if dt == FP4:
        # FP4 indexer queries (same passage): FP4 rows of dI/2 + dI/16 bytes per
        # head, decoded exactly (at most 6 significant bits, within binary32's
        # range) like the keys, which must then be FP4 rows too
        if kdt != FP4 or ka.shape[-1] != qa.shape[-1] or (qa.shape[-1] * 16) % 9:
            raise TypeError("FP4 queries need FP4 keys of the same row width")
        dI = qa.shape[-1] * 16 // 9
        qa = decode_rows(qa, dI).astype(np.float32)
        dt = F32
    if kdt == FP4:
        # FP4 indexer keys (same page, the passage on V4's FP4 indexer q/K): the
        # decoded values (at most 6 significant bits) are exact in fp32, and so
        # are the bf16 or fp32 queries; the formula is then the fp32 one
        dI = qa.shape[-1]
        ka = decode_rows(ka, dI).astype(np.float32)
        if qa.dtype == np.uint16:
            qa = (qa.astype(np.uint32) << 16).view(np.float32)
        dt = kdt = F32
    if kdt != dt:
        raise TypeError("qI and kI must share a dtype")
    wa = _f32(w)
    B, Q, HI, dI = qa.shape
    N = ka.shape[1]
    if ka.shape != (B, N, dI) or wa.shape != (B, Q, HI):
        raise ValueError("bad shapes")
    qp = _i64(q_pos)
    ca = _i32(cand)
    P = ca.shape[-1] if ca is not None else 0
    n = P if ca is not None else N
    out = np.empty((B, Q, n), dtype=np.float64)
    _lib().ora_index_score(_ptr(qa), _ptr(wa), _ptr(ka), dt, B, Q, HI, dI, N, _ptr(qp), m, _ptr(ca), P, _ptr(out))
    return out


# --------------------------------------------------------------- selection

def round_bf16(x) -> np.ndarray:
    """binary64 values rounded once to bfloat16 (nearest, ties to even), as float64.

    "读完这篇，你就搞懂 DeepSeek v4 了", the FP4 quantization-aware training
    passage: the indexer's score is quantized only down to BF16 for the top-k
    ranking (reading and method in the C file)."""
    a = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    out = np.empty_like(a)
    _lib().ora_round_bf16_array(_ptr(a), int(a.size), _ptr(out))
    return out


SCORE_KEYS = ("f64", "bf16")


def topk(scores, k: int, cand=None, key: str = "f64"):
    """Top-k per query: (idx int32 [..., k] ascending and -1 padded, count int32 [...]).

    Order by (score descending, entry index ascending); the k most relevant
    entries are kept ("闪电索引机制（对应步骤二）"), lowest index winning ties.
    key = "bf16": the ranked score is the binary64 score rounded to bfloat16
    (round_bf16), so scores that round alike tie and the lower index wins.
    """
    if key not in SCORE_KEYS:
        raise ValueError(key)
    s = np.ascontiguousarray(np.asarray(scores, dtype=np.float64))
    if key == "bf16":
        s = round_bf16(s)
    lead = s.shape[:-1]
    n = s.shape[-1]
    BQ = int(np.prod(lead)) if lead else 1
    ca = _i32(cand)
    if ca is not None and ca.shape != s.shape:
        raise ValueError("cand must match scores")
    idx = np.empty((BQ, k), dtype=np.int32)
    cnt = np.empty((BQ,), dtype=np.int32)
    _lib().ora_topk(_ptr(s), BQ, n, _ptr(ca), k, _ptr(idx), _ptr(cnt))
    return idx.reshape(*lead, k), cnt.reshape(lead)


# --------------------------------------------------------------- attention

def sparse_attn(q, kv, idx, scale: float, D: int | None = None):
    """Shared-KV sparse attention: (out float64 [B,Q,H,D], lse float64 [B,Q,H]).

    "读完这篇，你就搞懂 DeepSeek v4 了", section "注意力计算（对应步骤三）", eq. (9):
    standard softmax attention of every query head over the selected entries,
    one shared matrix C serving as both keys and values.
    """
    qa, qdt = _raw(q)
    ka, kdt = _raw(kv)
    B, Q, H, Dq = qa.shape
    D = Dq if D is None else D
    if D != Dq:
        raise ValueError("D mismatch")
    N = ka.shape[1]
    ia = _i32(idx)
    k = ia.shape[-1]
    if ia.shape != (B, Q, k):
        raise ValueError("idx must be [B,Q,k]")
    out = np.empty((B, Q, H, D), dtype=np.float64)
    lse = np.empty((B, Q, H), dtype=np.float64)
    _lib().ora_sparse_attn(_ptr(qa), qdt, _ptr(ka), kdt, B, Q, H, D, N, _ptr(ia), k, float(scale),
                           _ptr(out), _ptr(lse))
    return out, lse


# -------------------------------------------------------------- SWA branch

def window_idx(q_pos, W: int) -> np.ndarray:
    """Sliding-window entry list [B,Q,W] int32: positions p - W + 1 .. p of the
    query's own token and the W - 1 before it, ascending, -1 below 0.

    Video transcript on V4.1 Flash (prism.simon-ai.net), passages on the SWA
    branch: a 128-token window per layer, uncompressed, not shared across
    layers.  Reading: the query's own token is the newest of the W.
    """
    qp = _i64(q_pos)
    idx = np.empty(qp.shape + (W,), dtype=np.int32)
    _lib().ora_window_idx(_ptr(qp), int(qp.size), int(W), _ptr(idx))
    return idx


def merge_attn(o_a, lse_a, o_b, lse_b):
    """(out, lse) of one softmax over the union of two disjoint entry sets,
    from each set's attention output and log-sum-exp (all float64).

    Reading (the pages give no rule for combining the SWA and CSA2 branches):
    both sets enter a single softmax, so each branch is weighted by its share
    exp(lse) of the joint denominator.
    """
    oa = np.ascontiguousarray(o_a, dtype=np.float64)
    ob = np.ascontiguousarray(o_b, dtype=np.float64)
    la = np.ascontiguousarray(lse_a, dtype=np.float64)
    lb = np.ascontiguousarray(lse_b, dtype=np.float64)
    if oa.shape != ob.shape or la.shape != lb.shape or oa.shape[:-1] != la.shape:
        raise ValueError("shape mismatch")
    D = oa.shape[-1]
    out = np.empty_like(oa)
    lse = np.empty_like(la)
    _lib().ora_merge_attn(_ptr(oa), _ptr(la), _ptr(ob), _ptr(lb), int(la.size), int(D), _ptr(out), _ptr(lse))
    return out, lse


def swa_attn(q, swa_kv, q_pos, W: int, scale: float):
    """The sliding-window branch: shared-KV attention of every query head over
    the layer's own uncompressed window rows (the same row form as the global
    KV, one vector per token used as key and value)."""
    return sparse_attn(q, swa_kv, window_idx(q_pos, W), scale)


# ------------------------------------------------------------------- modes

def layer(mode: str, *, k: int, scale: float, q, kv, qI=None, w=None, kI=None, q_pos=None, m: int = 1,
          P: int = 0, pool=None, idx=None, score_key: str = "f64"):
    """One CSA2 layer in the given mode; returns a dict of outputs.

    Modes, per the V4.1 Flash transcript (prism.simon-ai.net) and "Recall之王
    祭出Reuse" (section "把KV Cache压到极致的几把杀手锏"):
      FULL    -- score every entry, keep top-k (and, with P > 0, the top-P
                 candidate pool), attend.
      REINDEX -- reuse the shared KV and indexer keys, score only the pool
                 with this layer's own queries, keep top-k of the pool, attend.
      REUSE   -- reuse KV and the previous top-k indices; attention only.
    score_key = "bf16" ranks (top-k and pool) by the scores rounded to bfloat16
    (see topk).
    """
    res = {}
    if mode == "FULL":
        s = index_score(qI, w, kI, q_pos=q_pos, m=m)
        res["scores"] = s
        res["idx"], res["count"] = topk(s, k, key=score_key)
        if P > 0:
            res["pool"], res["pool_count"] = topk(s, P, key=score_key)
    elif mode == "REINDEX":
        if pool is None:
            raise ValueError("REINDEX needs the pool")
        s = index_score(qI, w, kI, q_pos=q_pos, m=m, cand=pool)
        res["scores"] = s
        res["idx"], res["count"] = topk(s, k, cand=pool, key=score_key)
    elif mode == "REUSE":
        if idx is None:
            raise ValueError("REUSE needs the previous indices")
        res["idx"] = np.asarray(idx, dtype=np.int32)
    else:
        raise ValueError(mode)
    res["out"], res["lse"] = sparse_attn(q, kv, res["idx"], scale)
    return res


def default_scale(D: int) -> float:
    """Softmax scale 1/sqrt(D) (the tiny configuration fixes 1/sqrt(128) for D = 128)."""
    return 1.0 / math.sqrt(D)


def threads() -> int:
    """OpenMP threads the oracle will use (OMP_NUM_THREADS or the affinity mask)."""
    env = os.environ.get("OMP_NUM_THREADS")
    if env and env.isdigit():
        return int(env)
    return len(os.sched_getaffinity(0))
