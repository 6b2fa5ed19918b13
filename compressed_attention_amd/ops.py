"""Torch-facing wrappers of the libhattn C ABI.

Argument marshalling only: every step runs in the HIP kernels of
libhattn.so, on the caller's current stream.  Tensors must be contiguous
CUDA tensors; floating inputs are all fp32 or all bf16 (indexer head weights
and compression logits are always fp32).  See include/hattn.h for the exact
definition of each operation.
"""
from __future__ import annotations

import ctypes
import math

import torch

from ._lib import check, lib

_DT = {torch.float32: 0, torch.bfloat16: 1}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(dev) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a CUDA (HIP) device; there is no CPU path")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")


def _shape(t: torch.Tensor, name: str, shape) -> None:
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must be shaped {list(shape)}, got {list(t.shape)}")


def _on(dev, *named) -> None:
    """Every given tensor must sit on the device the call runs on."""
    for name, t in named:
        if t is not None and t.device != dev:
            raise ValueError(f"{name} is on {t.device}; the call runs on {dev}")


def _fdt(t: torch.Tensor, name: str) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"{name} must be float32 or bfloat16")
    return _DT[t.dtype]


# One workspace per (device, stream, purpose), grown on demand.  Calls on one
# stream are ordered, so they may share it; the torch caching allocator keeps
# a replaced buffer alive until the stream has passed its last use.
_WS: dict = {}


def _workspace(key, nbytes: int, device) -> torch.Tensor:
    t = _WS.get(key)
    if t is None or t.numel() < nbytes:
        t = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _WS[key] = t
    return t


def _ws_call(fn_name: str, key, device, call):
    """Runs a C call twice: size query (ws=NULL), then with the workspace."""
    sz = ctypes.c_size_t(0)
    check(fn_name, call(None, ctypes.byref(sz)))
    if sz.value == 0:
        check(fn_name, call(None, None))
        return
    ws = _workspace(key, sz.value, device)
    have = ctypes.c_size_t(ws.numel())
    check(fn_name, call(_ptr(ws), ctypes.byref(have)))


def compress(x, logits, pos_bias, w: int, stride: int, e_begin: int = 0, e_end: int | None = None, out=None):
    """Softmax-weighted window merge: x [bt][L][C] -> [bt][N][C] (x's dtype)."""
    _need(x, "x", ndim=3)
    dt = _fdt(x, "x")
    bt, L, C = x.shape
    N = (L - w) // stride + 1 if L >= w else 0
    if logits is not None:
        _need(logits, "logits", torch.float32, 2)
        if tuple(logits.shape) != (bt, L):
            raise ValueError("logits must be [bt][L]")
    if pos_bias is not None:
        _need(pos_bias, "pos_bias", torch.float32, 1)
        if pos_bias.numel() != w:
            raise ValueError("pos_bias must have w elements")
    if e_end is None:
        e_end = N
    if out is None:
        out = torch.empty((bt, N, C), dtype=x.dtype, device=x.device)
    else:
        _need(out, "out", x.dtype, 3)
        if tuple(out.shape) != (bt, N, C):
            raise ValueError(f"out must be [{bt}][{N}][{C}]")
    _on(x.device, ("logits", logits), ("pos_bias", pos_bias), ("out", out))
    check("hattn_compress", lib().hattn_compress(dt, _ptr(x), bt, L, C, _ptr(logits), _ptr(pos_bias), w, stride,
                                                 e_begin, e_end, _ptr(out), _stream(x.device)))
    return out


def compress_with_index(x, x_i, logits, pos_bias, w: int, stride: int, e_begin: int = 0, e_end: int | None = None,
                        out=None, out_i=None):
    """Compressed K|V entries and their indexer keys, both merged with each
    entry's own softmax weights: x [bt][L][C], x_i [bt][L][C_i] ->
    ([bt][N][C], [bt][N][C_i])."""
    _need(x, "x", ndim=3)
    dt = _fdt(x, "x")
    _need(x_i, "x_i", x.dtype, 3)
    bt, L, C = x.shape
    if tuple(x_i.shape[:2]) != (bt, L):
        raise ValueError("x_i must be [bt][L][C_i]")
    C_i = x_i.shape[2]
    N = (L - w) // stride + 1 if L >= w else 0
    if logits is not None:
        _need(logits, "logits", torch.float32, 2)
        _shape(logits, "logits", (bt, L))
    if pos_bias is not None:
        _need(pos_bias, "pos_bias", torch.float32, 1)
        _shape(pos_bias, "pos_bias", (w,))
    if e_end is None:
        e_end = N
    out = torch.empty((bt, N, C), dtype=x.dtype, device=x.device) if out is None else out
    out_i = torch.empty((bt, N, C_i), dtype=x.dtype, device=x.device) if out_i is None else out_i
    _need(out, "out", x.dtype, 3)
    _need(out_i, "out_i", x.dtype, 3)
    _shape(out, "out", (bt, N, C))
    _shape(out_i, "out_i", (bt, N, C_i))
    _on(x.device, ("x_i", x_i), ("logits", logits), ("pos_bias", pos_bias), ("out", out), ("out_i", out_i))
    check("hattn_compress_with_index",
          lib().hattn_compress_with_index(dt, _ptr(x), _ptr(x_i), bt, L, C, C_i, _ptr(logits), _ptr(pos_bias), w,
                                          stride, e_begin, e_end, _ptr(out), _ptr(out_i), _stream(x.device)))
    return out, out_i


def compress_channel_logits(x, logits, pos_bias, w: int, stride: int, e_begin: int = 0, e_end: int | None = None,
                            out=None):
    """Compression with one logit per raw token and channel: x [bt][L][C],
    logits [bt][L][C] fp32 -> [bt][N][C]."""
    _need(x, "x", ndim=3)
    dt = _fdt(x, "x")
    bt, L, C = x.shape
    _need(logits, "logits", torch.float32, 3)
    if tuple(logits.shape) != (bt, L, C):
        raise ValueError("logits must be [bt][L][C]")
    if pos_bias is not None:
        _need(pos_bias, "pos_bias", torch.float32, 1)
        _shape(pos_bias, "pos_bias", (w,))
    N = (L - w) // stride + 1 if L >= w else 0
    if e_end is None:
        e_end = N
    out = torch.empty((bt, N, C), dtype=x.dtype, device=x.device) if out is None else out
    _need(out, "out", x.dtype, 3)
    _shape(out, "out", (bt, N, C))
    _on(x.device, ("logits", logits), ("pos_bias", pos_bias), ("out", out))
    check("hattn_compress_channel_logits",
          lib().hattn_compress_channel_logits(dt, _ptr(x), bt, L, C, _ptr(logits), _ptr(pos_bias), w, stride, e_begin,
                                              e_end, _ptr(out), _stream(x.device)))
    return out


def visible_count(pos, w: int, stride: int, n_entries: int, out=None):
    """Entries visible at each raw position: int32 tensor shaped like pos."""
    _need(pos, "pos", torch.int32)
    if out is None:
        out = torch.empty_like(pos)
    _need(out, "out", torch.int32)
    _shape(out, "out", pos.shape)
    _on(pos.device, ("out", out))
    check("hattn_visible_count", lib().hattn_visible_count(_ptr(pos), pos.numel(), w, stride, n_entries, _ptr(out),
                                                           _stream(pos.device)))
    return out


def decode_append(x, logits, pos_bias, w: int, stride: int, q_pos, ckv, k_i=None, reps=None, B: int = 1,
                  n_vis=None, L: int | None = None):
    """Per-token maintenance of one compressed layer for a decode step (one
    query per sequence at q_pos [bt][1]): returns n_vis [bt][1]; rewrites the
    entry of ckv that the token completes and, with k_i / reps, the mean of
    the HISA block holding it.  With L given and x [bt][R][C] shorter than
    L, x and logits are rings of the newest R raw rows (row r at r % R)."""
    _need(x, "x", ndim=3)
    dt = _fdt(x, "x")
    bt, rows, C = x.shape
    L = rows if L is None else L
    raw_rows = 0 if rows == L else rows
    _need(q_pos, "q_pos", torch.int32)
    if q_pos.numel() != bt:
        raise ValueError("q_pos must hold one position per sequence")
    N = (L - w) // stride + 1 if L >= w else 0
    _need(ckv, "ckv", x.dtype, 3)
    if tuple(ckv.shape) != (bt, N, C):
        raise ValueError(f"ckv must be [{bt}][{N}][{C}]")
    if logits is not None:
        _need(logits, "logits", torch.float32)
        _shape(logits, "logits", (bt, rows))
    if pos_bias is not None:
        _need(pos_bias, "pos_bias", torch.float32)
        _shape(pos_bias, "pos_bias", (w,))
    d_i = 0
    if k_i is not None or reps is not None:
        _need(k_i, "k_i", x.dtype, 3)
        _need(reps, "reps", torch.float32, 3)
        d_i = k_i.shape[2]
        if k_i.shape[:2] != (bt, N) or tuple(reps.shape) != (bt, -(-N // B), d_i):
            raise ValueError("k_i must be [bt][N][d_i] and reps [bt][ceil(N/B)][d_i]")
    if n_vis is None:
        n_vis = torch.empty(q_pos.shape, dtype=torch.int32, device=x.device)
    _need(n_vis, "n_vis", torch.int32)
    _shape(n_vis, "n_vis", q_pos.shape)
    _on(x.device, ("logits", logits), ("pos_bias", pos_bias), ("q_pos", q_pos), ("ckv", ckv), ("k_i", k_i),
        ("reps", reps), ("n_vis", n_vis))
    check("hattn_decode_append", lib().hattn_decode_append(dt, _ptr(x), bt, L, raw_rows, C, _ptr(logits),
                                                           _ptr(pos_bias), w, stride, _ptr(q_pos), _ptr(ckv),
                                                           _ptr(n_vis), _ptr(k_i), d_i, B, _ptr(reps),
                                                           _stream(x.device)))
    return n_vis


def _index_common(q_i, k_i, w_i, n_vis):
    _need(q_i, "q_i", ndim=4)
    dt = _fdt(q_i, "q_i")
    _need(k_i, "k_i", q_i.dtype, 3)
    _need(w_i, "w_i", torch.float32, 3)
    _need(n_vis, "n_vis", torch.int32, 2)
    bt, nq, h_i, d_i = q_i.shape
    if k_i.shape[0] != bt or k_i.shape[2] != d_i or tuple(w_i.shape) != (bt, nq, h_i) or tuple(n_vis.shape) != (bt, nq):
        raise ValueError("indexer shapes disagree")
    _on(q_i.device, ("k_i", k_i), ("w_i", w_i), ("n_vis", n_vis))
    return dt, bt, nq, h_i, d_i, k_i.shape[1]


def index_topk(q_i, k_i, w_i, n_vis, k: int, return_scores: bool = False):
    """Flat indexer: idx [bt][nq][k] int32 (ascending, -1 padded)."""
    dt, bt, nq, h_i, d_i, n = _index_common(q_i, k_i, w_i, n_vis)
    idx = torch.empty((bt, nq, k), dtype=torch.int32, device=q_i.device)
    sc = torch.empty((bt, nq, k), dtype=torch.float32, device=q_i.device) if return_scores else None
    L = lib()
    st = _stream(q_i.device)

    def call(ws, szp):
        return L.hattn_index_topk(dt, _ptr(q_i), _ptr(k_i), _ptr(w_i), _ptr(n_vis), bt, nq, h_i, d_i, n, k,
                                  _ptr(idx), _ptr(sc), ws, szp, st)

    _ws_call("hattn_index_topk", ("index", q_i.device, st.value), q_i.device, call)
    return (idx, sc) if return_scores else idx


def hisa_pool(k_i, B: int, j_begin: int = 0, j_end: int | None = None, out=None):
    """Block means of k_i [bt][n][d_i] -> fp32 [bt][ceil(n/B)][d_i]."""
    _need(k_i, "k_i", ndim=3)
    dt = _fdt(k_i, "k_i")
    bt, n, d_i = k_i.shape
    nb = -(-n // B)
    if j_end is None:
        j_end = nb
    if out is None:
        out = torch.empty((bt, nb, d_i), dtype=torch.float32, device=k_i.device)
    else:
        _need(out, "out", torch.float32, 3)
        _shape(out, "out", (bt, nb, d_i))
        _on(k_i.device, ("out", out))
    check("hattn_hisa_pool", lib().hattn_hisa_pool(dt, _ptr(k_i), bt, n, d_i, B, j_begin, j_end, _ptr(out),
                                                   _stream(k_i.device)))
    return out


def hisa_topk(q_i, k_i, w_i, n_vis, reps, B: int, m: int, k: int, return_blocks: bool = False):
    """Two-stage HISA selection: idx [bt][nq][k] (and blocks [bt][nq][m])."""
    dt, bt, nq, h_i, d_i, n = _index_common(q_i, k_i, w_i, n_vis)
    _need(reps, "reps", torch.float32, 3)
    if tuple(reps.shape) != (bt, -(-n // B), d_i):
        raise ValueError("reps must be [bt][ceil(n/B)][d_i]")
    _on(q_i.device, ("reps", reps))
    idx = torch.empty((bt, nq, k), dtype=torch.int32, device=q_i.device)
    blk = torch.empty((bt, nq, m), dtype=torch.int32, device=q_i.device) if return_blocks else None
    L = lib()
    st = _stream(q_i.device)

    def call(ws, szp):
        return L.hattn_hisa_topk(dt, _ptr(q_i), _ptr(k_i), _ptr(w_i), _ptr(n_vis), bt, nq, h_i, d_i, n, _ptr(reps),
                                 B, m, k, _ptr(idx), _ptr(blk), ws, szp, st)

    _ws_call("hattn_hisa_topk", ("hisa", q_i.device, st.value), q_i.device, call)
    return (idx, blk) if return_blocks else idx


def block_sparse_topk(q_i, k_i, w_i, n_vis, reps, B: int, m: int, return_blocks: bool = False):
    """Block-sparse baseline: every visible entry of the top-m blocks (HISA's
    block choice): idx [bt][nq][m*B] (and blocks [bt][nq][m])."""
    dt, bt, nq, h_i, d_i, n = _index_common(q_i, k_i, w_i, n_vis)
    _need(reps, "reps", torch.float32, 3)
    if tuple(reps.shape) != (bt, -(-n // B), d_i):
        raise ValueError("reps must be [bt][ceil(n/B)][d_i]")
    _on(q_i.device, ("reps", reps))
    idx = torch.empty((bt, nq, m * B), dtype=torch.int32, device=q_i.device)
    blk = torch.empty((bt, nq, m), dtype=torch.int32, device=q_i.device) if return_blocks else None
    L = lib()
    st = _stream(q_i.device)

    def call(ws, szp):
        return L.hattn_block_sparse_topk(dt, _ptr(q_i), _ptr(k_i), _ptr(w_i), _ptr(n_vis), bt, nq, h_i, d_i, n,
                                         _ptr(reps), B, m, _ptr(idx), _ptr(blk), ws, szp, st)

    _ws_call("hattn_block_sparse_topk", ("hisa", q_i.device, st.value), q_i.device, call)
    return (idx, blk) if return_blocks else idx


def _ring_rows(raw_kv, L):
    """(L, raw_rows) for the attention calls: raw_kv [bt][R][2d] with L given
    and R < L is a ring of the newest R raw rows (row r at slot r % R)."""
    rows = raw_kv.shape[1]
    L = rows if L is None else L
    return L, (0 if rows == L else rows)


def _attn_common(q, ckv, raw_kv, q_pos):
    _need(q, "q", ndim=4)
    dt = _fdt(q, "q")
    _need(ckv, "ckv", q.dtype, 3)
    _need(raw_kv, "raw_kv", q.dtype, 3)
    _need(q_pos, "q_pos", torch.int32, 2)
    bt, nq, h, d = q.shape
    if ckv.shape[0] != bt or ckv.shape[2] != 2 * d or raw_kv.shape[0] != bt or raw_kv.shape[2] != 2 * d:
        raise ValueError("K|V rows must be [.., 2*d]")
    if tuple(q_pos.shape) != (bt, nq):
        raise ValueError("q_pos must be [bt][nq]")
    _on(q.device, ("ckv", ckv), ("raw_kv", raw_kv), ("q_pos", q_pos))
    return dt, bt, nq, h, d


def sparse_attn(q, ckv, idx, raw_kv, q_pos, window: int, scale: float | None = None, return_lse: bool = False,
                L: int | None = None):
    """Attention over ckv[idx] plus the raw window: out [bt][nq][h][d] fp32.
    With L given and raw_kv shorter than L, raw_kv is a ring of the newest
    raw rows (row r at slot r % R) that holds every row the queries read."""
    dt, bt, nq, h, d = _attn_common(q, ckv, raw_kv, q_pos)
    L_raw, raw_rows = _ring_rows(raw_kv, L)
    _need(idx, "idx", torch.int32, 3)
    if idx.shape[:2] != (bt, nq):
        raise ValueError("idx must be [bt][nq][k]")
    _on(q.device, ("idx", idx))
    k = idx.shape[2]
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = torch.empty((bt, nq, h, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((bt, nq, h), dtype=torch.float32, device=q.device) if return_lse else None
    lb = lib()
    st = _stream(q.device)

    def call(ws, szp):
        return lb.hattn_sparse_attn(dt, _ptr(q), _ptr(ckv), ckv.shape[1], _ptr(idx), k, _ptr(raw_kv), L_raw, raw_rows,
                                    _ptr(q_pos), window, scale, bt, nq, h, d, _ptr(out), _ptr(lse), ws, szp, st)

    _ws_call("hattn_sparse_attn", ("attn", q.device, st.value), q.device, call)
    return (out, lse) if return_lse else out


def sparse_attn_noalloc(q, ckv, idx, raw_kv, q_pos, window: int, scale: float | None = None, out=None, lse=None,
                        L: int | None = None):
    """sparse_attn through the entry point that allocates nothing (the
    library's static scratch instead of a workspace).  Pass out (and lse) to
    keep the call free of allocations on the torch side too."""
    dt, bt, nq, h, d = _attn_common(q, ckv, raw_kv, q_pos)
    L_raw, raw_rows = _ring_rows(raw_kv, L)
    _need(idx, "idx", torch.int32, 3)
    if idx.shape[:2] != (bt, nq):
        raise ValueError("idx must be [bt][nq][k]")
    _on(q.device, ("idx", idx))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    if out is None:
        out = torch.empty((bt, nq, h, d), dtype=torch.float32, device=q.device)
    _need(out, "out", torch.float32, 4)
    _shape(out, "out", (bt, nq, h, d))
    if lse is not None:
        _need(lse, "lse", torch.float32, 3)
        _shape(lse, "lse", (bt, nq, h))
    _on(q.device, ("out", out), ("lse", lse))
    check("hattn_sparse_attn_noalloc",
          lib().hattn_sparse_attn_noalloc(dt, _ptr(q), _ptr(ckv), ckv.shape[1], _ptr(idx), idx.shape[2], _ptr(raw_kv),
                                          L_raw, raw_rows, _ptr(q_pos), window, scale, bt, nq, h, d, _ptr(out),
                                          _ptr(lse), _stream(q.device)))
    return out


def dense_compressed_attn(q, ckv, n_vis, raw_kv, q_pos, window: int, scale: float | None = None,
                          return_lse: bool = False, L: int | None = None):
    """Attention over ckv[0 .. n_vis) plus the raw window: out [bt][nq][h][d]
    fp32 (raw_kv as in sparse_attn, a ring when L is given and longer)."""
    dt, bt, nq, h, d = _attn_common(q, ckv, raw_kv, q_pos)
    L_raw, raw_rows = _ring_rows(raw_kv, L)
    _need(n_vis, "n_vis", torch.int32, 2)
    _shape(n_vis, "n_vis", (bt, nq))
    _on(q.device, ("n_vis", n_vis))
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    out = torch.empty((bt, nq, h, d), dtype=torch.float32, device=q.device)
    lse = torch.empty((bt, nq, h), dtype=torch.float32, device=q.device) if return_lse else None
    lb = lib()
    st = _stream(q.device)

    def call(ws, szp):
        return lb.hattn_dense_compressed_attn(dt, _ptr(q), _ptr(ckv), ckv.shape[1], _ptr(n_vis), _ptr(raw_kv),
                                              L_raw, raw_rows, _ptr(q_pos), window, scale, bt, nq, h, d, _ptr(out),
                                              _ptr(lse), ws, szp, st)

    _ws_call("hattn_dense_compressed_attn", ("attn", q.device, st.value), q.device, call)
    return (out, lse) if return_lse else out


# ---- kernel timer -----------------------------------------------------------

def timer_enable(on: bool) -> None:
    check("hattn_timer_enable", lib().hattn_timer_enable(1 if on else 0))


def timer_collect() -> dict:
    """Waits for recorded launches; returns {kernel: (total_ms, count)}."""
    L = lib()
    check("hattn_timer_collect", L.hattn_timer_collect())
    buf = ctypes.create_string_buffer(1 << 16)
    check("hattn_timer_names", L.hattn_timer_names(buf, len(buf)))
    out = {}
    for name in filter(None, buf.value.decode().split("\n")):
        ms, cnt = ctypes.c_double(), ctypes.c_int64()
        check("hattn_timer_query", L.hattn_timer_query(name.encode(), ctypes.byref(ms), ctypes.byref(cnt)))
        out[name] = (ms.value, cnt.value)
    return out


class DecodePlan:
    """One decode step of a hybrid layer pair (CSA branch: cache append ->
    HISA -> sparse attention; HCA branch: cache append -> dense attention),
    validated once and run with one host call per step (hattn_decode_plan_*).

    Tensors are the per-step inputs of the separate ops with nq = 1: q_pos
    [bt][1]; csa_q / hca_q [bt][1][h][d]; q_i [bt][1][h_i][d_i]; w_i
    [bt][1][h_i].  csa_ckv, hca_ckv and reps are rewritten in place each run.
    The plan holds references to every tensor; outputs live in .csa_out /
    .hca_out ([bt][1][h][d] fp32), with return_lse in .csa_lse / .hca_lse,
    and with return_idx the CSA selection in .csa_idx ([bt][1][k] int32).
    """

    def __init__(self, *, q_pos, csa_raw_kv, csa_logits, csa_pos_bias, csa_ckv, k_i, reps, q_i, w_i, csa_q,
                 hca_raw_kv, hca_logits, hca_pos_bias, hca_ckv, hca_q, B: int, m: int, k: int, csa_w: int = 8,
                 csa_stride: int = 4, hca_w: int = 128, hca_stride: int = 128, window: int = 128,
                 scale: float | None = None, return_lse: bool = False, return_idx: bool = False,
                 L: int | None = None):
        from ._lib import DecodeDesc

        self._plan = None
        for name, t in [("csa_raw_kv", csa_raw_kv), ("csa_ckv", csa_ckv), ("k_i", k_i), ("q_i", q_i),
                        ("csa_q", csa_q), ("hca_raw_kv", hca_raw_kv), ("hca_ckv", hca_ckv), ("hca_q", hca_q)]:
            _need(t, name)
        dt = _fdt(csa_raw_kv, "csa_raw_kv")
        _need(q_pos, "q_pos", torch.int32)
        _need(reps, "reps", torch.float32, 3)
        _need(w_i, "w_i", torch.float32)
        bt, rows, C = csa_raw_kv.shape
        # with L given and fewer raw rows than L, the raw arrays are rings of
        # the newest rows (row r at slot r % rows)
        L = rows if L is None else L
        raw_rows = 0 if rows == L else rows
        h, d = csa_q.shape[-2], csa_q.shape[-1]
        if q_pos.numel() != bt or csa_q.numel() != bt * h * d or hca_q.numel() != bt * h * d:
            raise ValueError("one query per sequence: q_pos [bt][1], csa_q / hca_q [bt][1][h][d]")
        if C != 2 * d or tuple(hca_raw_kv.shape) != (bt, rows, C):
            raise ValueError("raw K|V rows must be [bt][rows][2d] for both branches")
        h_i, d_i = q_i.shape[-2], q_i.shape[-1]
        if q_i.numel() != bt * h_i * d_i or w_i.numel() != bt * h_i:
            raise ValueError("q_i must be [bt][1][h_i][d_i] and w_i [bt][1][h_i]")
        for name, t in [("csa_logits", csa_logits), ("csa_pos_bias", csa_pos_bias), ("hca_logits", hca_logits),
                        ("hca_pos_bias", hca_pos_bias)]:
            if t is not None:
                _need(t, name, torch.float32)
        # the caches the plan rewrites and reads, shaped as the layer
        # geometry implies (the library sees only their addresses)
        for name, t in [("csa_ckv", csa_ckv), ("hca_ckv", hca_ckv), ("hca_raw_kv", hca_raw_kv), ("csa_q", csa_q),
                        ("hca_q", hca_q), ("k_i", k_i), ("q_i", q_i)]:
            if t.dtype != csa_raw_kv.dtype:
                raise TypeError(f"{name} must be {csa_raw_kv.dtype}, got {t.dtype}")
        n_csa = (L - csa_w) // csa_stride + 1 if L >= csa_w else 0
        n_hca = (L - hca_w) // hca_stride + 1 if L >= hca_w else 0
        _shape(csa_ckv, "csa_ckv", (bt, n_csa, C))
        _shape(hca_ckv, "hca_ckv", (bt, n_hca, C))
        _shape(k_i, "k_i", (bt, n_csa, d_i))
        _shape(reps, "reps", (bt, -(-n_csa // B) if B > 0 else 0, d_i))
        for name, t, w in [("csa_logits", csa_logits, None), ("hca_logits", hca_logits, None),
                           ("csa_pos_bias", csa_pos_bias, csa_w), ("hca_pos_bias", hca_pos_bias, hca_w)]:
            if t is not None:
                _shape(t, name, (bt, rows) if w is None else (w,))
        dev = csa_raw_kv.device
        _on(dev, ("q_pos", q_pos), ("csa_logits", csa_logits), ("csa_pos_bias", csa_pos_bias), ("csa_ckv", csa_ckv),
            ("k_i", k_i), ("reps", reps), ("q_i", q_i), ("w_i", w_i), ("csa_q", csa_q), ("hca_raw_kv", hca_raw_kv),
            ("hca_logits", hca_logits), ("hca_pos_bias", hca_pos_bias), ("hca_ckv", hca_ckv), ("hca_q", hca_q))
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        self.csa_out = torch.empty((bt, 1, h, d), dtype=torch.float32, device=dev)
        self.hca_out = torch.empty((bt, 1, h, d), dtype=torch.float32, device=dev)
        self.csa_lse = torch.empty((bt, 1, h), dtype=torch.float32, device=dev) if return_lse else None
        self.hca_lse = torch.empty((bt, 1, h), dtype=torch.float32, device=dev) if return_lse else None
        self.csa_idx = torch.empty((bt, 1, k), dtype=torch.int32, device=dev) if return_idx else None
        self._keep = [q_pos, csa_raw_kv, csa_logits, csa_pos_bias, csa_ckv, k_i, reps, q_i, w_i, csa_q, hca_raw_kv,
                      hca_logits, hca_pos_bias, hca_ckv, hca_q]
        self.device = dev
        desc = DecodeDesc(dtype=dt, h=h, d=d, window=window, bt=bt, L=L, raw_rows=raw_rows, scale=scale, h_i=h_i,
                          d_i=d_i, B=B, m=m,
                          k=k, csa_w=csa_w, csa_stride=csa_stride, hca_w=hca_w, hca_stride=hca_stride,
                          q_pos=_ptr(q_pos), csa_raw_kv=_ptr(csa_raw_kv), csa_logits=_ptr(csa_logits),
                          csa_pos_bias=_ptr(csa_pos_bias), csa_ckv=_ptr(csa_ckv), k_i=_ptr(k_i), reps=_ptr(reps),
                          q_i=_ptr(q_i), w_i=_ptr(w_i), csa_q=_ptr(csa_q), csa_out=_ptr(self.csa_out),
                          csa_lse=_ptr(self.csa_lse), csa_idx=_ptr(self.csa_idx), hca_raw_kv=_ptr(hca_raw_kv), hca_logits=_ptr(hca_logits),
                          hca_pos_bias=_ptr(hca_pos_bias), hca_ckv=_ptr(hca_ckv), hca_q=_ptr(hca_q),
                          hca_out=_ptr(self.hca_out), hca_lse=_ptr(self.hca_lse), ws=None, ws_bytes=0)
        Lb = lib()
        sz = ctypes.c_size_t(0)
        check("hattn_decode_plan_ws_bytes", Lb.hattn_decode_plan_ws_bytes(ctypes.byref(desc), ctypes.byref(sz)))
        self._ws = torch.empty(max(sz.value, 256), dtype=torch.uint8, device=dev)
        desc.ws = self._ws.data_ptr()
        desc.ws_bytes = self._ws.numel()
        plan = ctypes.c_void_p()
        with torch.cuda.device(dev):
            check("hattn_decode_plan_create", Lb.hattn_decode_plan_create(ctypes.byref(desc), ctypes.byref(plan)))
        self._plan = plan
        self._run = Lb.hattn_decode_plan_run

    def run(self, stream=None):
        """Enqueues one step on `stream` (default: the current stream)."""
        st = ctypes.c_void_p((stream or torch.cuda.current_stream(self.device)).cuda_stream)
        status = self._run(self._plan, st)
        if status != 0:
            check("hattn_decode_plan_run", status)
        return self.csa_out, self.hca_out

    def run_graph(self, stream=None):
        """The same step as one launch of a HIP graph that the first call
        captures (hattn_decode_plan_run_graph)."""
        st = ctypes.c_void_p((stream or torch.cuda.current_stream(self.device)).cuda_stream)
        check("hattn_decode_plan_run_graph", lib().hattn_decode_plan_run_graph(self._plan, st))
        return self.csa_out, self.hca_out

    def close(self):
        if self._plan is not None:
            check("hattn_decode_plan_destroy", lib().hattn_decode_plan_destroy(self._plan))
            self._plan = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
