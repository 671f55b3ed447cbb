"""Python binding of libcsa2.so: argument marshalling only.

Every computation runs in the library's HIP kernels; this module checks tensor
dtypes/devices, allocates outputs and workspace with torch (device memory and
streams are torch's), and passes raw pointers and the current stream through
the C ABI declared in ``include/csa2.h``.  If the library is missing this
module raises ImportError: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa2.so")

F32, BF16, FP4, FP4QK = 0, 1, 2, 3
SCORE_FMTS = {"f64": 0, "bf16": 1}
FULL, REINDEX, REUSE = 0, 1, 2
MODES = {"FULL": FULL, "REINDEX": REINDEX, "REUSE": REUSE}
STATUS = {0: "CSA2_OK", 1: "CSA2_EINVAL", 2: "CSA2_EUNSUPPORTED", 3: "CSA2_EWORKSPACE", 4: "CSA2_EHIP",
          5: "CSA2_EINTERNAL"}

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python -m sparse_long_context_csa2_amd.build`")

_lib = ctypes.CDLL(LIB_PATH)

_vp, _i32, _i64, _f32, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t


class LayerArgs(ctypes.Structure):
    """Mirror of csa2_layer_args."""
    _fields_ = [
        ("mode", _i32), ("B", _i32), ("Q", _i32), ("N", _i64), ("m", _i32), ("HI", _i32), ("dI", _i32),
        ("idx_dt", _i32), ("k", _i32), ("P", _i32), ("H", _i32), ("D", _i32), ("q_dt", _i32), ("kv_dt", _i32),
        ("scale", _f32),
        ("q_pos", _vp), ("qI", _vp), ("w", _vp), ("kI", _vp), ("pool", _vp), ("idx", _vp), ("count", _vp),
        ("scores", _vp), ("q", _vp), ("kv", _vp), ("out", _vp), ("lse", _vp), ("score_fmt", _i32),
    ]


def _sig(name, res, args):
    f = getattr(_lib, name)
    f.restype, f.argtypes = res, args
    return f


_compress_ws = _sig("csa2_compress_workspace_size", _sz, [ctypes.c_int, _i64, _i32, _i32, _i32])
_compress = _sig("csa2_compress", ctypes.c_int, [_vp, ctypes.c_int, _i64, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz,
                                                 _vp])
_index_ws = _sig("csa2_index_score_workspace_size", _sz, [ctypes.c_int, _i32, _i32, _i32, _i32, _i64, _i32])
_index = _sig("csa2_index_score", ctypes.c_int, [_vp, _vp, _vp, ctypes.c_int, _i32, _i32, _i32, _i32, _i64, _vp, _i32,
                                                 _vp, _i32, _vp, _vp, _vp, _sz, _vp])
_topk_ws = _sig("csa2_topk_workspace_size", _sz, [_i32, _i32, _i64, _i32])
_topk = _sig("csa2_topk", ctypes.c_int, [_vp, _i32, _i32, _i64, _vp, _i32, _vp, _vp, _vp, _sz, _vp])
_attn_ws = _sig("csa2_sparse_attn_workspace_size", _sz, [ctypes.c_int, ctypes.c_int, _i32, _i32, _i32, _i32, _i32])
_attn = _sig("csa2_sparse_attn", ctypes.c_int, [_vp, _vp, ctypes.c_int, ctypes.c_int, _i32, _i32, _i32, _i32, _i64,
                                                _vp, _i32, _f32, _vp, _vp, _vp, _sz, _vp])
_swa_ws = _sig("csa2_swa_attn_workspace_size", _sz, [ctypes.c_int, ctypes.c_int, _i32, _i32, _i32, _i32, _i32])
_swa = _sig("csa2_swa_attn", ctypes.c_int, [_vp, _vp, ctypes.c_int, ctypes.c_int, _i32, _i32, _i32, _i32, _i64, _vp,
                                            _i32, _f32, _vp, _vp, _vp, _vp, _vp, _sz, _vp])
_quant = _sig("csa2_quantize_fp4", ctypes.c_int, [_vp, ctypes.c_int, _i64, _i32, _vp, _vp, _vp])
_merge = _sig("csa2_merge_attn", ctypes.c_int, [_vp, _vp, _vp, _vp, ctypes.c_int, _i64, _i32, _vp, _vp, _vp])
_layer_ws = _sig("csa2_layer_workspace_size", _sz, [ctypes.POINTER(LayerArgs)])
_ws_alias = _sig("csa2_workspace_size", _sz, [ctypes.POINTER(LayerArgs)])
_layer = _sig("csa2_layer", ctypes.c_int, [ctypes.POINTER(LayerArgs), _vp, _sz, _vp])
_layer_noalloc = _sig("csa2_layer_noalloc", ctypes.c_int, [ctypes.POINTER(LayerArgs), _vp])
NOALLOC_SCRATCH_BYTES = 64 << 20
_last_error = _sig("csa2_last_error", ctypes.c_char_p, [])
_version = _sig("csa2_version", ctypes.c_char_p, [])

EXPORTS = ["csa2_compress_workspace_size", "csa2_compress", "csa2_index_score_workspace_size", "csa2_index_score",
           "csa2_topk_workspace_size", "csa2_topk", "csa2_sparse_attn_workspace_size", "csa2_sparse_attn",
           "csa2_swa_attn_workspace_size", "csa2_swa_attn", "csa2_merge_attn", "csa2_quantize_fp4",
           "csa2_layer_workspace_size", "csa2_workspace_size", "csa2_layer", "csa2_layer_noalloc", "csa2_last_error",
           "csa2_version"]


class Csa2Error(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{STATUS.get(code, code)}: {msg}")
        self.code = code


def version() -> str:
    return _version().decode()


def _check(rc):
    if rc != 0:
        raise Csa2Error(rc, _last_error().decode())


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dt(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.uint8:
        return FP4
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(*ts):
    for t in ts:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("tensors must be on the GPU")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def _workspace(nbytes, device, ws=None):
    if nbytes == 0:
        return None
    if ws is not None and ws.numel() >= nbytes:
        return ws
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def kv_row_width(kv, D=None):
    """Channels D of a stored KV tensor (FP4 rows: D/2 + D/16 bytes)."""
    if kv.dtype == torch.uint8:
        return kv.shape[-1] * 16 // 9 if D is None else D
    return kv.shape[-1]


# ------------------------------------------------------------ entry points

def compress(x, n_out, m, halo, wz, bias, out=None, ws=None):
    _dev(x, wz, bias)
    D = x.shape[-1]
    dt = _dt(x)
    if out is None:
        out = torch.empty(n_out, D, dtype=x.dtype, device=x.device)
    nws = _compress_ws(dt, n_out, D, m, halo)
    wsb = _workspace(nws, x.device, ws)
    _check(_compress(_p(x), dt, n_out, D, m, halo, _p(wz), _p(bias), _p(out), _p(wsb), nws, _stream()))
    return out


def _index_shape(qI, kI):
    """(B, Q, HI, dI, dtype code) of indexer inputs: FP4 keys (uint8 rows) with
    bf16 queries, FP4 queries and keys (both uint8 rows), or plain tensors."""
    if qI.dtype == torch.uint8:
        if kI.dtype != torch.uint8 or qI.shape[-1] != kI.shape[-1] or (qI.shape[-1] * 16) % 9:
            raise TypeError("FP4 queries need FP4 keys of the same row width")
        B, Q, HI, rb = qI.shape
        return B, Q, HI, rb * 16 // 9, FP4QK
    B, Q, HI, dI = qI.shape
    return B, Q, HI, dI, (FP4 if kI.dtype == torch.uint8 else _dt(qI))


def index_score(qI, w, kI, q_pos=None, m=1, cand=None, want_err=True, scores=None, ws=None):
    _dev(qI, w, kI, q_pos, cand)
    B, Q, HI, dI, dt = _index_shape(qI, kI)
    N = kI.shape[1]
    P = cand.shape[-1] if cand is not None else 0
    n = P if cand is not None else N
    if scores is None:
        scores = torch.empty(B, Q, n, dtype=torch.float32, device=qI.device)
    err = torch.empty(B, Q, dtype=torch.float32, device=qI.device) if want_err else None
    nws = _index_ws(dt, B, Q, HI, dI, N, P)
    wsb = _workspace(nws, qI.device, ws)
    _check(_index(_p(qI), _p(w), _p(kI), dt, B, Q, HI, dI, N, _p(q_pos), m, _p(cand), P, _p(scores), _p(err),
                  _p(wsb), nws, _stream()))
    return scores, err


def topk(scores, k, cand=None, ws=None):
    _dev(scores, cand)
    B, Q, n = scores.shape
    idx = torch.empty(B, Q, k, dtype=torch.int32, device=scores.device)
    count = torch.empty(B, Q, dtype=torch.int32, device=scores.device)
    nws = _topk_ws(B, Q, n, k)
    wsb = _workspace(nws, scores.device, ws)
    _check(_topk(_p(scores), B, Q, n, _p(cand), k, _p(idx), _p(count), _p(wsb), nws, _stream()))
    return idx, count


def sparse_attn(q, kv, idx, scale, D=None, want_lse=True, out=None, ws=None):
    _dev(q, kv, idx)
    B, Q, H, Dq = q.shape
    D = Dq if D is None else D
    N = kv.shape[1]
    k = idx.shape[-1]
    q_dt, kv_dt = _dt(q), _dt(kv)
    if out is None:
        out = torch.empty(B, Q, H, D, dtype=q.dtype, device=q.device)
    lse = torch.empty(B, Q, H, dtype=torch.float32, device=q.device) if want_lse else None
    nws = _attn_ws(q_dt, kv_dt, B, Q, H, D, k)
    wsb = _workspace(nws, q.device, ws)
    _check(_attn(_p(q), _p(kv), q_dt, kv_dt, B, Q, H, D, N, _p(idx), k, scale, _p(out), _p(lse), _p(wsb), nws,
                 _stream()))
    return out, lse


def quantize_fp4(x, cache=None, dst_row=None):
    """FP4 rows of x [n, D] (fp32/bf16) written into cache rows dst_row (int64
    [n]; rows 0..n-1 when None).  cache: uint8 [rows, D/2 + D/16], allocated
    for n rows when None."""
    _dev(x, cache, dst_row)
    n, D = x.shape
    if cache is None:
        cache = torch.empty(n, D // 2 + D // 16, dtype=torch.uint8, device=x.device)
    _check(_quant(_p(x), _dt(x), n, D, _p(cache), _p(dst_row), _stream()))
    return cache


def swa_attn(q, swa_kv, q_pos, W, scale, csa_out=None, csa_lse=None, want_lse=True, out=None, ws=None):
    """The sliding-window branch over the layer's own rows swa_kv [B,T,row]
    (window p - W + 1 .. p of each query position), merged with the CSA2
    branch's (csa_out, csa_lse) when given.  out may be csa_out."""
    _dev(q, swa_kv, q_pos, csa_out, csa_lse)
    B, Q, H, D = q.shape
    T = swa_kv.shape[1]
    q_dt, kv_dt = _dt(q), _dt(swa_kv)
    if out is None:
        out = torch.empty(B, Q, H, D, dtype=q.dtype, device=q.device)
    lse = torch.empty(B, Q, H, dtype=torch.float32, device=q.device) if want_lse else None
    nws = _swa_ws(q_dt, kv_dt, B, Q, H, D, W)
    wsb = _workspace(nws, q.device, ws)
    _check(_swa(_p(q), _p(swa_kv), q_dt, kv_dt, B, Q, H, D, T, _p(q_pos), W, scale, _p(csa_out), _p(csa_lse),
                _p(out), _p(lse), _p(wsb), nws, _stream()))
    return out, lse


def merge_attn(o_a, lse_a, o_b, lse_b, out=None, want_lse=True):
    """One softmax over the union of two disjoint entry sets from each set's
    attention output [..., D] and lse [...]."""
    _dev(o_a, lse_a, o_b, lse_b)
    D = o_a.shape[-1]
    R = lse_a.numel()
    if out is None:
        out = torch.empty_like(o_a)
    lse = torch.empty_like(lse_a) if want_lse else None
    _check(_merge(_p(o_a), _p(lse_a), _p(o_b), _p(lse_b), _dt(o_a), R, D, _p(out), _p(lse), _stream()))
    return out, lse


class Layer:
    """One prepared csa2_layer call: outputs and workspace allocated once, so
    ``run()`` only launches (graph-capturable, no allocation)."""

    def __init__(self, mode, *, q, kv, k=None, scale, qI=None, w=None, kI=None, q_pos=None, m=1, P=0, pool=None,
                 idx=None, keep_scores=False, want_lse=True, count=True, out=None, noalloc=False, score_fmt="f64"):
        mode_i = MODES[mode] if isinstance(mode, str) else mode
        _dev(q, kv, qI, w, kI, q_pos, pool, idx, out)
        B, Q, H, D = q.shape
        dev = q.device
        # the library takes k and P as the row strides of idx and pool: tensors
        # given by the caller must have exactly those shapes
        if mode_i == REUSE and idx is not None and k is None:
            k = idx.shape[-1]
        if idx is not None and tuple(idx.shape) != (B, Q, k):
            raise ValueError(f"idx has shape {tuple(idx.shape)}, expected {(B, Q, k)}")
        if pool is not None and mode_i == FULL and tuple(pool.shape) != (B, Q, P):
            raise ValueError(f"pool has shape {tuple(pool.shape)}, expected {(B, Q, P)}")
        if pool is not None and (pool.dim() != 3 or tuple(pool.shape[:2]) != (B, Q)):
            raise ValueError(f"pool has shape {tuple(pool.shape)}, expected ({B}, {Q}, P)")
        if out is not None and tuple(out.shape) != tuple(q.shape):
            raise ValueError(f"out has shape {tuple(out.shape)}, expected {tuple(q.shape)}")
        for name, t in (("idx", idx), ("pool", pool)):
            if t is not None and t.dtype != torch.int32:
                raise TypeError(f"{name} must be int32")
        if kv.dim() != 3 or kv.shape[0] != B:
            raise ValueError(f"kv has shape {tuple(kv.shape)}, expected ({B}, N, row)")
        a = LayerArgs()
        a.mode, a.B, a.Q, a.N, a.m = mode_i, B, Q, kv.shape[1], m
        a.H, a.D, a.q_dt, a.kv_dt, a.scale, a.k = H, D, _dt(q), _dt(kv), float(scale), k
        self.tensors = {"q": q, "kv": kv}
        if mode_i != REUSE:
            _, _, a.HI, a.dI, a.idx_dt = _index_shape(qI, kI)
            a.score_fmt = SCORE_FMTS[score_fmt]
            self.tensors.update(qI=qI, w=w, kI=kI, q_pos=q_pos)
            if mode_i == FULL:
                a.P = P
                if P > 0 and pool is None:
                    pool = torch.empty(B, Q, P, dtype=torch.int32, device=dev)
            else:
                if pool is None:
                    raise ValueError("REINDEX needs the pool")
                a.P = pool.shape[-1]
            if idx is None:
                idx = torch.empty(B, Q, k, dtype=torch.int32, device=dev)
            n = kv.shape[1] if mode_i == FULL else a.P
            self.scores = torch.empty(B, Q, n, dtype=torch.float32, device=dev) if keep_scores else None
        else:
            if idx is None:
                raise ValueError("REUSE needs the previous indices")
            self.scores = None
        self.pool, self.idx = pool, idx
        self.count = torch.empty(B, Q, dtype=torch.int32, device=dev) if (count and mode_i != REUSE) else None
        self.out = out if out is not None else torch.empty(B, Q, H, D, dtype=q.dtype, device=dev)
        self.lse = torch.empty(B, Q, H, dtype=torch.float32, device=dev) if want_lse else None
        a.q_pos, a.qI, a.w, a.kI = _p(q_pos), _p(qI), _p(w), _p(kI)
        a.pool, a.idx, a.count, a.scores = _p(pool), _p(idx), _p(self.count), _p(self.scores)
        a.q, a.kv, a.out, a.lse = _p(q), _p(kv), _p(self.out), _p(self.lse)
        self.args = a
        self.noalloc = noalloc
        self.ws_bytes = 0 if noalloc else _layer_ws(ctypes.byref(a))
        self.ws = None if noalloc else _workspace(self.ws_bytes, dev)

    def set_query(self, q):
        """Point the layer at a new query tensor of the same shape (no copy)."""
        _dev(q)
        self.tensors["q"] = q
        self.args.q = _p(q)

    def run(self):
        if self.noalloc:  # csa2_layer_noalloc: the library's own scratch, no workspace
            _check(_layer_noalloc(ctypes.byref(self.args), _stream()))
        else:
            _check(_layer(ctypes.byref(self.args), _p(self.ws), self.ws_bytes, _stream()))
        return self


def layer(mode, **kw):
    """Run one CSA2 layer; returns a dict with idx, count, pool, scores, out, lse."""
    L = Layer(mode, **kw).run()
    return {"idx": L.idx, "count": L.count, "pool": L.pool, "scores": L.scores, "out": L.out, "lse": L.lse}
