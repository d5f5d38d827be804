"""Python binding of libdsa, the MI355X (gfx950) sparse MQA attention step.

Every function here only marshals torch tensors into the C ABI of
`include/dsa.h` (pointers, sizes, the current HIP stream) and allocates
outputs with torch; all arithmetic happens in the HIP kernels.  If the shared
library is missing, importing this package raises: there is no fallback.

Calls (same names as the C entry points):
    dsa_index_scores  scores of every compressed row per query
    dsa_topk          the index_topk best visible rows per query
    dsa_window_idx    sliding-window part of each index row
    dsa_sparse_attn   attention with a per-head sink over the indexed rows
    dsa_sparse_attn_select  the index rows and the attention (one launch for decode batches)
    dsa_sparse_attn_step    the whole step: index scores, index rows, attention (one launch
                            for decode batches)
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_F32, DSA_BF16 = 0, 1
DSA_KV_DENSE, DSA_KV_FP4_E4M3_G16 = 0, 1
_ERRORS = {-1: "NULL", -2: "SHAPE", -3: "DTYPE", -4: "UNSUPPORTED", -5: "HIP", -6: "WORKSPACE"}


class DsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"DSA_ERR_{_ERRORS.get(code, code)}: {msg}")
        self.code = code


class DsaKvSrc(ctypes.Structure):
    _fields_ = [
        ("rows", ctypes.c_void_p),
        ("n_rows", ctypes.c_int64),
        ("batch_stride", ctypes.c_int64),
        ("row_stride", ctypes.c_int64),
        ("format", ctypes.c_int),
        ("scales", ctypes.c_void_p),
        ("scale_batch_stride", ctypes.c_int64),
        ("scale_row_stride", ctypes.c_int64),
    ]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, f32 = ctypes.c_int, ctypes.c_int64, ctypes.c_void_p, ctypes.c_float
    lib.dsa_abi_version.restype = i32
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_index_scores.argtypes = [vp, vp, i64, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.dsa_index_scores.restype = i32
    lib.dsa_topk.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, i64, vp]
    lib.dsa_topk.restype = i32
    lib.dsa_select.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, i64, vp]
    lib.dsa_select.restype = i32
    lib.dsa_window_idx.argtypes = [i32, i32, i32, i32, vp, i64, vp]
    lib.dsa_window_idx.restype = i32
    lib.dsa_window_cols.argtypes = [i32, i32, i32]
    lib.dsa_window_cols.restype = i32
    lib.dsa_sparse_attn.argtypes = [vp, ctypes.POINTER(DsaKvSrc), ctypes.POINTER(DsaKvSrc), vp, vp, i32, f32, vp,
                                    i32, i32, i32, i32, i32, vp, ctypes.c_size_t, vp]
    lib.dsa_sparse_attn.restype = i32
    lib.dsa_sparse_attn_select.argtypes = [vp, i32, i32, i32, i32, i32, vp, ctypes.POINTER(DsaKvSrc),
                                           ctypes.POINTER(DsaKvSrc), vp, f32, vp, i32, i32, i32, i32, i32, vp, vp,
                                           ctypes.c_size_t, vp]
    lib.dsa_sparse_attn_select.restype = i32
    lib.dsa_sparse_attn_step.argtypes = [vp, vp, i64, vp, f32, i32, i32, i32, i32, i32, i32, i32, vp,
                                         ctypes.POINTER(DsaKvSrc), ctypes.POINTER(DsaKvSrc), vp, f32, vp, i32, i32,
                                         i32, i32, i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.dsa_sparse_attn_step.restype = i32
    lib.dsa_sparse_attn_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
    lib.dsa_sparse_attn_workspace_size.restype = ctypes.c_size_t
    return lib


lib = _load()
ABI_VERSION = lib.dsa_abi_version()


def _check(rc: int) -> None:
    if rc != 0:
        raise DsaError(rc, lib.dsa_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return DSA_F32
    if t.dtype == torch.bfloat16:
        return DSA_BF16
    raise DsaError(-3, f"dtype {t.dtype} is not float32/bfloat16")


def _dev(*ts) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        if t.device != dev or dev.type != "cuda":
            raise DsaError(-2, "all tensors must be on the same GPU")
    return dev


def _stream(dev, stream):
    s = torch.cuda.current_stream(dev) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need_contig(name, t):
    if not t.is_contiguous():
        raise DsaError(-2, f"{name} must be contiguous")


def _batched_rows(name, t):
    """(batch_stride, row_stride) in elements of a [B, n, D] view with unit inner stride."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise DsaError(-2, f"{name} must be [B, n, row] with contiguous rows")
    return t.stride(0), t.stride(1)


# --------------------------------------------------------------------------- calls
def dsa_index_scores(q_idx, k_idx, w, w_scale: float, start_pos: int, ratio: int, out=None, stream=None):
    """Index scores [B, S, T] float32; see `dsa_index_scores` in include/dsa.h.

    q_idx [B,S,H_I,D_I], k_idx [B,T,D_I] (any batch stride), w [B,S,H_I] (same dtype).
    """
    dev = _dev(q_idx, k_idx, w)
    _need_contig("q_idx", q_idx)
    _need_contig("w", w)
    B, S, H, Dd = q_idx.shape
    T = k_idx.shape[1]
    kbs, krs = _batched_rows("k_idx", k_idx)
    if krs != Dd:
        raise DsaError(-2, "k_idx rows must be dense")
    if out is None:
        out = torch.empty(B, S, T, dtype=torch.float32, device=dev)
    _need_contig("scores", out)
    _check(lib.dsa_index_scores(_ptr(q_idx), _ptr(k_idx), kbs, _ptr(w), float(w_scale), _dtype_code(q_idx), B, S, T,
                                H, Dd, int(start_pos), int(ratio), _ptr(out), _stream(dev, stream)))
    return out


def dsa_topk(scores, index_topk: int, start_pos: int, ratio: int, offset: int, out=None, col: int = 0,
             stream=None):
    """Top-k index rows; writes K = min(index_topk, T) columns of `out` [B,S,>=col+K] from `col` on."""
    dev = _dev(scores)
    _need_contig("scores", scores)
    B, S, T = scores.shape
    K = min(int(index_topk), T)
    if out is None:
        out = torch.empty(B, S, col + K, dtype=torch.int32, device=dev)
    _need_contig("idx", out)
    if out.dtype != torch.int32 or out.shape[-1] < col + K:
        raise DsaError(-2, "idx must be int32 with room for the top-k columns")
    base = ctypes.c_void_p(out.data_ptr() + 4 * col)
    _check(lib.dsa_topk(_ptr(scores), B, S, T, int(index_topk), int(start_pos), int(ratio), int(offset), base,
                        out.shape[-1], _stream(dev, stream)))
    return out


def dsa_window_cols(S: int, start_pos: int, W: int) -> int:
    n = lib.dsa_window_cols(int(S), int(start_pos), int(W))
    if n < 0:
        _check(n)
    return n


def dsa_window_idx(out, start_pos: int, W: int, stream=None):
    """Window index rows into the first window columns of `out` [B, S, >=Wc] int32."""
    dev = _dev(out)
    _need_contig("idx", out)
    B, S, ld = out.shape
    _check(lib.dsa_window_idx(B, S, int(start_pos), int(W), _ptr(out), ld, _stream(dev, stream)))
    return out


def dsa_select(scores, index_topk: int, start_pos: int, ratio: int, W: int, offset: int, out=None, stream=None):
    """Whole index rows [B, S, Wc + K]: window columns, then the top-k columns (one launch)."""
    B, S, T = scores.shape
    dev = _dev(scores)
    _need_contig("scores", scores)
    Wc = dsa_window_cols(S, start_pos, W)
    K = min(int(index_topk), T)
    if out is None:
        out = torch.empty(B, S, Wc + K, dtype=torch.int32, device=dev)
    _need_contig("idx", out)
    if out.dtype != torch.int32 or out.shape[-1] < Wc + K:
        raise DsaError(-2, "idx must be int32 with room for the window and top-k columns")
    _check(lib.dsa_select(_ptr(scores), B, S, T, int(index_topk), int(start_pos), int(ratio), int(W), int(offset),
                          _ptr(out), out.shape[-1], _stream(dev, stream)))
    return out


def kv_src(rows, scales=None, fmt: int = DSA_KV_DENSE) -> DsaKvSrc:
    """Describe one KV source: rows [B, n, D] (dense) or [B, n, D/2] uint8 with scales [B, n, D/16] (fp4)."""
    src = DsaKvSrc()
    if rows is None:
        return src
    bs, rs = _batched_rows("kv rows", rows)
    src.rows = rows.data_ptr()
    src.n_rows = rows.shape[1]
    src.batch_stride = bs
    src.row_stride = rs
    src.format = fmt
    if fmt == DSA_KV_FP4_E4M3_G16:
        sbs, srs = _batched_rows("kv scales", scales)
        src.scales = scales.data_ptr()
        src.scale_batch_stride = sbs
        src.scale_row_stride = srs
    return src


def dsa_sparse_attn_workspace_size(dtype_code: int, B: int, S: int, H: int, D: int, L: int) -> int:
    return int(lib.dsa_sparse_attn_workspace_size(dtype_code, B, S, H, D, L))


def dsa_sparse_attn(q, kv_win, kv_comp, sink, idx, scale: float, comp_scales=None, out=None, workspace=None,
                    stream=None):
    """Sparse attention with a per-head sink; o [B,S,H,D] in q's dtype.

    kv_win [B, n_win, D]; kv_comp [B, T, D] in q's dtype, or [B, T, D/2] uint8 fp4 nibbles with
    comp_scales [B, T, D/16] uint8 E4M3; idx [B, S, L] int32 over [window rows | compressed rows].
    """
    dev = _dev(q, kv_win, kv_comp, sink, idx)
    _need_contig("q", q)
    _need_contig("idx", idx)
    B, S, H, D = q.shape
    L = idx.shape[-1]
    dt = _dtype_code(q)
    win = kv_src(kv_win)
    fp4 = kv_comp is not None and kv_comp.dtype == torch.uint8
    comp = kv_src(kv_comp, comp_scales, DSA_KV_FP4_E4M3_G16 if fp4 else DSA_KV_DENSE)
    if out is None:
        out = torch.empty_like(q)
    _need_contig("o", out)
    need = dsa_sparse_attn_workspace_size(dt, B, S, H, D, L)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_attn(_ptr(q), ctypes.byref(win), ctypes.byref(comp), _ptr(sink), _ptr(idx), L,
                               float(scale), _ptr(out), dt, B, S, H, D, _ptr(workspace), wbytes,
                               _stream(dev, stream)))
    return out


def dsa_sparse_attn_select(scores, q, kv_win, kv_comp, sink, *, index_topk: int, start_pos: int, ratio: int,
                           W: int, scale: float, comp_scales=None, out=None, idx=None, workspace=None, stream=None):
    """Index rows (window + top-k, as dsa_select with offset kv_win.shape[1]) and the sparse attention
    over them; one launch for decode batches the two-phase decode kernel takes.  Returns (o, idx);
    idx [B, S, L] int32 receives the rows (allocated when not given)."""
    dev = _dev(q, kv_win, kv_comp, sink, scores)
    _need_contig("q", q)
    _need_contig("scores", scores)
    B, S, H, D = q.shape
    T = scores.shape[-1]
    Wc = dsa_window_cols(S, start_pos, W)
    L = Wc + min(int(index_topk), T)
    dt = _dtype_code(q)
    win = kv_src(kv_win)
    fp4 = kv_comp is not None and kv_comp.dtype == torch.uint8
    comp = kv_src(kv_comp, comp_scales, DSA_KV_FP4_E4M3_G16 if fp4 else DSA_KV_DENSE)
    if out is None:
        out = torch.empty_like(q)
    _need_contig("o", out)
    if idx is None:
        idx = torch.empty(B, S, L, dtype=torch.int32, device=dev)
    _need_contig("idx", idx)
    if idx.dtype != torch.int32 or idx.shape[-1] != L:
        raise DsaError(-2, "idx must be int32 [B, S, L] with L = window columns + top-k columns")
    need = dsa_sparse_attn_workspace_size(dt, B, S, H, D, L)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_attn_select(_ptr(scores), T, int(index_topk), int(start_pos), int(ratio), int(W), _ptr(q),
                                      ctypes.byref(win), ctypes.byref(comp), _ptr(sink), float(scale), _ptr(out), dt,
                                      B, S, H, D, _ptr(idx), _ptr(workspace), wbytes, _stream(dev, stream)))
    return out, idx


def dsa_sparse_attn_step(q_idx, k_idx, w, q, kv_win, kv_comp, sink, *, index_topk: int, start_pos: int, ratio: int,
                         W: int, scale: float, w_scale: float, comp_scales=None, out=None, scores=None, idx=None,
                         workspace=None, stream=None):
    """The whole step: index scores (as dsa_index_scores), index rows and the sparse attention over
    them (as dsa_sparse_attn_select); one launch for decode batches the decode kernel takes.
    Returns (o, idx, scores); scores [B, S, T] float32 and idx [B, S, L] int32 are allocated when not
    given."""
    dev = _dev(q_idx, k_idx, w, q, kv_win, kv_comp, sink)
    _need_contig("q_idx", q_idx)
    _need_contig("w", w)
    _need_contig("q", q)
    B, S, H, D = q.shape
    H_I, D_I = q_idx.shape[2], q_idx.shape[3]
    T = k_idx.shape[1]
    kbs, krs = _batched_rows("k_idx", k_idx)
    if krs != D_I:
        raise DsaError(-2, "k_idx rows must be dense")
    Wc = dsa_window_cols(S, start_pos, W)
    L = Wc + min(int(index_topk), T)
    dt = _dtype_code(q)
    win = kv_src(kv_win)
    fp4 = kv_comp is not None and kv_comp.dtype == torch.uint8
    comp = kv_src(kv_comp, comp_scales, DSA_KV_FP4_E4M3_G16 if fp4 else DSA_KV_DENSE)
    if out is None:
        out = torch.empty_like(q)
    _need_contig("o", out)
    if scores is None:
        scores = torch.empty(B, S, T, dtype=torch.float32, device=dev)
    _need_contig("scores", scores)
    if idx is None:
        idx = torch.empty(B, S, L, dtype=torch.int32, device=dev)
    _need_contig("idx", idx)
    if idx.dtype != torch.int32 or idx.shape[-1] != L:
        raise DsaError(-2, "idx must be int32 [B, S, L] with L = window columns + top-k columns")
    need = dsa_sparse_attn_workspace_size(dt, B, S, H, D, L)
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_attn_step(_ptr(q_idx), _ptr(k_idx), kbs, _ptr(w), float(w_scale), H_I, D_I, T,
                                    int(index_topk), int(start_pos), int(ratio), int(W), _ptr(q), ctypes.byref(win),
                                    ctypes.byref(comp), _ptr(sink), float(scale), _ptr(out), dt, B, S, H, D,
                                    _ptr(scores), _ptr(idx), _ptr(workspace), wbytes, _stream(dev, stream)))
    return out, idx, scores


def sparse_attention_step(q, kv_win, kv_comp, qI, kI, w, sink, *, start_pos: int, ratio: int, W: int,
                          index_topk: int, scale: float, w_scale: float, comp_scales=None, bufs=None,
                          stream=None):
    """One pass of the whole step: window rows, index scores, top-k, sparse attention.

    Returns (o, idx, scores).  `bufs` may carry preallocated 'scores', 'idx', 'o', 'workspace'.
    """
    bufs = {} if bufs is None else bufs
    B, S = q.shape[:2]
    T = kI.shape[1]
    Wc = dsa_window_cols(S, start_pos, W)
    K = min(index_topk, T)
    idx = bufs.get("idx")
    if idx is None:
        idx = torch.empty(B, S, Wc + K, dtype=torch.int32, device=q.device)
    if T > 0:
        return dsa_sparse_attn_step(qI, kI, w, q, kv_win, kv_comp, sink, index_topk=index_topk, start_pos=start_pos,
                                    ratio=ratio, W=W, scale=scale, w_scale=w_scale, comp_scales=comp_scales,
                                    out=bufs.get("o"), scores=bufs.get("scores"), idx=idx,
                                    workspace=bufs.get("workspace"), stream=stream)
    dsa_window_idx(idx, start_pos, W, stream=stream)
    o = dsa_sparse_attn(q, kv_win, None, sink, idx, scale, out=bufs.get("o"), workspace=bufs.get("workspace"),
                        stream=stream)
    return o, idx, bufs.get("scores")


__all__ = [
    "DsaError",
    "DsaKvSrc",
    "dsa_index_scores",
    "dsa_topk",
    "dsa_select",
    "dsa_window_cols",
    "dsa_window_idx",
    "dsa_sparse_attn",
    "dsa_sparse_attn_select",
    "dsa_sparse_attn_step",
    "dsa_sparse_attn_workspace_size",
    "kv_src",
    "sparse_attention_step",
    "lib",
    "ABI_VERSION",
]
