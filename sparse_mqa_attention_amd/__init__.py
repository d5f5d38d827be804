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
    dsa_init, dsa_device_errors, dsa_last_launches, dsa_set_debug, dsa_check_idx, dsa_topk_plan
                            set-up, error flags and introspection

The library is set up for a device (dsa_init) the first time a call here uses it.  Workspaces
are allocated zero-filled, as the C ABI asks.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

DSA_F32, DSA_BF16 = 0, 1
DSA_KV_DENSE, DSA_KV_FP4_E4M3_G16 = 0, 1
_ERRORS = {-1: "NULL", -2: "SHAPE", -3: "DTYPE", -4: "UNSUPPORTED", -5: "HIP", -6: "WORKSPACE", -7: "STATE",
           -8: "INDEX"}


class DsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"DSA_ERR_{_ERRORS.get(code, code)}: {msg}")
        self.code = code


class DsaCandidates(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_void_p), ("ld_bits", ctypes.c_int64), ("block_size", ctypes.c_int)]


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
    lib.dsa_last_launch_count.restype = i32
    lib.dsa_last_launches.restype = ctypes.c_char_p
    lib.dsa_init.argtypes = [i32]
    lib.dsa_init.restype = i32
    lib.dsa_device_errors.argtypes = [i32, ctypes.POINTER(ctypes.c_uint32)]
    lib.dsa_device_errors.restype = i32
    lib.dsa_set_debug.argtypes = [i32]
    lib.dsa_set_debug.restype = i32
    lib.dsa_check_idx.argtypes = [vp, i64, i64, ctypes.POINTER(ctypes.c_int64)]
    lib.dsa_check_idx.restype = i32
    lib.dsa_topk_plan.argtypes = [i32, i32, i32, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    lib.dsa_topk_plan.restype = i32
    lib.dsa_index_scores.argtypes = [vp, vp, i64, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32, vp, vp]
    lib.dsa_index_scores.restype = i32
    lib.dsa_index_scores_mxfp4.argtypes = [vp, vp, vp, vp, i64, vp, f32, i32, i32, i32, i32, i32, i32, i32,
                                           ctypes.POINTER(DsaCandidates), vp, vp]
    lib.dsa_index_scores_masked.argtypes = [vp, vp, i64, vp, f32, i32, i32, i32, i32, i32, i32, i32, i32,
                                            ctypes.POINTER(DsaCandidates), vp, vp]
    lib.dsa_index_scores_masked.restype = i32
    lib.dsa_candidate_blocks.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, i64, vp]
    lib.dsa_candidate_blocks.restype = i32
    lib.dsa_index_scores_mxfp4.restype = i32
    lib.dsa_sparse_attn_step_mxfp4.argtypes = [vp, vp, vp, vp, i64, vp, f32, i32, i32, i32, i32, i32, i32, i32, vp,
                                               ctypes.POINTER(DsaKvSrc), ctypes.POINTER(DsaKvSrc), vp, f32, vp, i32,
                                               i32, i32, i32, i32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.dsa_sparse_attn_step_mxfp4.restype = i32
    lib.dsa_topk.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, vp, i64, vp, ctypes.c_size_t, vp]
    lib.dsa_topk.restype = i32
    lib.dsa_topk_workspace_size.argtypes = [i32, i32, i32, i32]
    lib.dsa_topk_workspace_size.restype = ctypes.c_size_t
    lib.dsa_select.argtypes = [vp, i32, i32, i32, i32, i32, i32, i32, i32, vp, i64, vp, ctypes.c_size_t, vp]
    lib.dsa_select.restype = i32
    lib.dsa_step_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32, i32, i32, i32]
    lib.dsa_step_workspace_size.restype = ctypes.c_size_t
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
    lib.dsa_sparse_attn_step_noalloc.argtypes = [vp, vp, i64, vp, f32, i32, i32, i32, i32, i32, i32, i32, vp,
                                                 ctypes.POINTER(DsaKvSrc), ctypes.POINTER(DsaKvSrc), vp, f32, vp,
                                                 i32, i32, i32, i32, i32, vp, vp, vp]
    lib.dsa_sparse_attn_step_noalloc.restype = i32
    lib.dsa_sparse_attn_rope.argtypes = [vp, ctypes.POINTER(DsaKvSrc), ctypes.POINTER(DsaKvSrc), vp, vp, i32, f32, vp,
                                         i32, i32, i32, i32, i32, vp, i32, vp, ctypes.c_size_t, vp]
    lib.dsa_sparse_attn_rope.restype = i32
    lib.dsa_rope_inverse.argtypes = [vp, i32, i32, i32, i32, i32, vp, i32, vp]
    lib.dsa_rope_inverse.restype = i32
    lib.dsa_compress_kv_write.argtypes = [vp, i64, i32, i32, i32, vp, i32, vp, i64, vp, i64, i64, vp]
    lib.dsa_compress_kv_write.restype = i32
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


_READY = set()  # device indices dsa_init has prepared


def dsa_init(device=None) -> None:
    """Per-device set-up of the library (dsa_init in include/dsa.h); idempotent."""
    d = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    i = d.index if d.index is not None else torch.cuda.current_device()
    if i in _READY:
        return
    _check(lib.dsa_init(i))
    _READY.add(i)


def _dev(*ts) -> torch.device:
    dev = ts[0].device
    for t in ts:
        if t is None:
            continue
        if t.device != dev or dev.type != "cuda":
            raise DsaError(-2, "all tensors must be on the same GPU")
    if dev.index not in _READY:
        dsa_init(dev)
    return dev


def dsa_last_launches():
    """(count, names) of the kernels the last call on this thread launched."""
    return int(lib.dsa_last_launch_count()), lib.dsa_last_launches().decode()


def dsa_device_errors(device=None) -> int:
    """Read and clear the device's sticky error bits (synchronises the device)."""
    i = torch.cuda.current_device() if device is None else torch.device(device).index
    v = ctypes.c_uint32(0)
    _check(lib.dsa_device_errors(i, ctypes.byref(v)))
    return int(v.value)


def dsa_set_debug(on: bool) -> bool:
    return bool(lib.dsa_set_debug(1 if on else 0))


def dsa_check_idx(idx_host, n_rows: int):
    """Host-side range check of an int32 numpy array: (ok, first bad position or -1)."""
    import numpy as np

    a = np.ascontiguousarray(idx_host, dtype=np.int32)
    bad = ctypes.c_int64(-1)
    rc = lib.dsa_check_idx(a.ctypes.data_as(ctypes.c_void_p), a.size, int(n_rows), ctypes.byref(bad))
    if rc not in (0, -8):
        _check(rc)
    return rc == 0, int(bad.value)


def dsa_topk_plan(B: int, S: int, T: int):
    """(rows on the one-wave kernel, rows on the per-row workgroup kernel) of a top-k call."""
    w, b = ctypes.c_int64(0), ctypes.c_int64(0)
    _check(lib.dsa_topk_plan(int(B), int(S), int(T), ctypes.byref(w), ctypes.byref(b)))
    return int(w.value), int(b.value)


def _expect(name, t, shape, dtype):
    if t is None:
        raise DsaError(-1, f"{name} is missing")
    if tuple(t.shape) != tuple(shape):
        raise DsaError(-2, f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise DsaError(-3, f"{name} has dtype {t.dtype}, expected {dtype}")


def _workspace(need, workspace, dev):
    if need and (workspace is None or workspace.numel() * workspace.element_size() < need):
        workspace = torch.zeros(need, dtype=torch.uint8, device=dev)  # the header must start at zero
    return workspace


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
    _need_contig("q_idx", q_idx)
    _need_contig("w", w)
    B, S, H, Dd = q_idx.shape
    T = k_idx.shape[1]
    kbs, krs = _batched_rows("k_idx", k_idx)
    if krs != Dd or k_idx.shape[0] != B or k_idx.shape[2] != Dd:
        raise DsaError(-2, "k_idx must be [B, T, D_I] with dense rows")
    _expect("k_idx", k_idx, (B, T, Dd), q_idx.dtype)
    _expect("w", w, (B, S, H), q_idx.dtype)
    if out is not None:
        _expect("scores", out, (B, S, T), torch.float32)
    dev = _dev(q_idx, k_idx, w, out)
    if out is None:
        out = torch.empty(B, S, T, dtype=torch.float32, device=dev)
    _expect("scores", out, (B, S, T), torch.float32)
    _need_contig("scores", out)
    _check(lib.dsa_index_scores(_ptr(q_idx), _ptr(k_idx), kbs, _ptr(w), float(w_scale), _dtype_code(q_idx), B, S, T,
                                H, Dd, int(start_pos), int(ratio), _ptr(out), _stream(dev, stream)))
    return out


def _mx_index_operands(qI, qI_scale, kI, kI_scale, w):
    """Shapes of MXFP4 index operands, checked: (B, S, H_I, D_I, T, k_batch_rows)."""
    for name, t in (("qI", qI), ("qI_scale", qI_scale), ("kI", kI), ("kI_scale", kI_scale)):
        if t is None or t.dtype != torch.uint8:
            raise DsaError(-3, f"{name} must be uint8 (packed e2m1 nibbles / E8M0 scale bytes)")
    _need_contig("qI", qI)
    _need_contig("qI_scale", qI_scale)
    if qI.dim() != 4 or kI.dim() != 3:
        raise DsaError(-2, "qI must be [B, S, H_I, D_I/2] and kI [B, T, D_I/2]")
    B, S, H, half = qI.shape
    D_I = 2 * half
    T = kI.shape[1]
    _expect("qI_scale", qI_scale, (B, S, H, D_I // 32), torch.uint8)
    if kI.shape[0] != B or kI.shape[2] != half or kI.stride(2) != 1 or kI.stride(1) != half:
        raise DsaError(-2, "kI must be [B, T, D_I/2] with dense rows")
    if tuple(kI_scale.shape) != (B, T, D_I // 32) or kI_scale.stride(2) != 1 or kI_scale.stride(1) != D_I // 32:
        raise DsaError(-2, "kI_scale must be [B, T, D_I/32] with dense rows")
    rows = kI.stride(0) // half
    if kI.stride(0) % half or kI_scale.stride(0) != rows * (D_I // 32):
        raise DsaError(-2, "kI and kI_scale must be slices of caches with the same row count per batch")
    if w.dtype != torch.bfloat16:
        raise DsaError(-3, "w must be bfloat16")
    _expect("w", w, (B, S, H), torch.bfloat16)
    _need_contig("w", w)
    return B, S, H, D_I, T, rows


def _cand(candidates, B, S, T):
    """The C descriptor of a (bits [B, S, words] int32/uint32 tensor, block_size) pair, or NULL."""
    if candidates is None:
        return None
    bits, bs = candidates
    if bits.dim() != 3 or tuple(bits.shape[:2]) != (B, S) or bits.element_size() != 4 or bits.stride(2) != 1:
        raise DsaError(-2, "candidate bits must be a [B, S, words] tensor of 32-bit words")
    if bits.stride(1) != bits.shape[2] or bits.stride(0) != S * bits.shape[2]:
        raise DsaError(-2, "candidate bits must be contiguous")
    c = DsaCandidates()
    c.bits = bits.data_ptr()
    c.ld_bits = bits.shape[2]
    c.block_size = int(bs)
    return c


def dsa_candidate_blocks(scores, start_pos: int, ratio: int, block_size: int, n_blocks: int, out=None, stream=None):
    """Candidate blocks of the two-level selection (dsa_candidate_blocks): int32 bit words
    [B, S, ceil(ceil(T / block_size) / 32)], bit i of a row set when block i is chosen."""
    _need_contig("scores", scores)
    if scores.dtype != torch.float32 or scores.dim() != 3:
        raise DsaError(-3, "scores must be float32 [B, S, T]")
    B, S, T = scores.shape
    words = ((T + block_size - 1) // block_size + 31) // 32
    if out is not None:
        _expect("candidate bits", out, (B, S, words), torch.int32)
    dev = _dev(scores, out)
    if out is None:
        out = torch.empty(B, S, words, dtype=torch.int32, device=dev)
    _check(lib.dsa_candidate_blocks(_ptr(scores), B, S, T, int(start_pos), int(ratio), int(block_size),
                                    int(n_blocks), _ptr(out), words, _stream(dev, stream)))
    return out


def dsa_index_scores_masked(q_idx, k_idx, w, w_scale: float, start_pos: int, ratio: int, candidates, out=None,
                            stream=None):
    """dsa_index_scores with candidate blocks (bits, block_size) from dsa_candidate_blocks: -inf outside them."""
    _need_contig("q_idx", q_idx)
    _need_contig("w", w)
    B, S, H, Dd = q_idx.shape
    T = k_idx.shape[1]
    kbs, krs = _batched_rows("k_idx", k_idx)
    if krs != Dd:
        raise DsaError(-2, "k_idx rows must be dense")
    _expect("k_idx", k_idx, (B, T, Dd), q_idx.dtype)
    _expect("w", w, (B, S, H), q_idx.dtype)
    if out is not None:
        _expect("scores", out, (B, S, T), torch.float32)
    cand = _cand(candidates, B, S, T)
    dev = _dev(q_idx, k_idx, w, out, None if candidates is None else candidates[0])
    if out is None:
        out = torch.empty(B, S, T, dtype=torch.float32, device=dev)
    _check(lib.dsa_index_scores_masked(_ptr(q_idx), _ptr(k_idx), kbs, _ptr(w), float(w_scale), _dtype_code(q_idx), B,
                                       S, T, H, Dd, int(start_pos), int(ratio),
                                       None if cand is None else ctypes.byref(cand), _ptr(out), _stream(dev, stream)))
    return out


def dsa_index_scores_mxfp4(qI, qI_scale, kI, kI_scale, w, w_scale: float, start_pos: int, ratio: int, out=None,
                           candidates=None, stream=None):
    """Index scores [B, S, T] float32 from MXFP4 index operands; see `dsa_index_scores_mxfp4` in
    include/dsa.h.  qI [B,S,H_I,D_I/2] uint8, qI_scale [B,S,H_I,D_I/32] uint8, kI [B,T,D_I/2] uint8,
    kI_scale [B,T,D_I/32] uint8 (cache slices allowed), w [B,S,H_I] bf16."""
    B, S, H, D_I, T, rows = _mx_index_operands(qI, qI_scale, kI, kI_scale, w)
    if out is not None:
        _expect("scores", out, (B, S, T), torch.float32)
    cand = _cand(candidates, B, S, T)
    dev = _dev(qI, qI_scale, kI, kI_scale, w, out, None if candidates is None else candidates[0])
    if out is None:
        out = torch.empty(B, S, T, dtype=torch.float32, device=dev)
    _need_contig("scores", out)
    _check(lib.dsa_index_scores_mxfp4(_ptr(qI), _ptr(qI_scale), _ptr(kI), _ptr(kI_scale), rows, _ptr(w),
                                      float(w_scale), B, S, T, H, D_I, int(start_pos), int(ratio),
                                      None if cand is None else ctypes.byref(cand), _ptr(out),
                                      _stream(dev, stream)))
    return out


def dsa_sparse_attn_step_mxfp4(qI, qI_scale, kI, kI_scale, w, q, kv_win, kv_comp, sink, *, index_topk: int,
                               start_pos: int, ratio: int, W: int, scale: float, w_scale: float, comp_scales=None,
                               out=None, scores=None, idx=None, workspace=None, stream=None):
    """The whole step with MXFP4 index operands (dsa_sparse_attn_step_mxfp4): returns (o, idx, scores)."""
    B, S, H_I, D_I, T, rows = _mx_index_operands(qI, qI_scale, kI, kI_scale, w)
    Bq, Sq, H, D, dt, win, comp, out = _attn_operands(q, kv_win, kv_comp, sink, comp_scales, out)
    if (Bq, Sq) != (B, S):
        raise DsaError(-2, "q and the index queries disagree on [B, S]")
    Wc = dsa_window_cols(S, start_pos, W)
    L = Wc + min(int(index_topk), T)
    if scores is not None:
        _expect("scores", scores, (B, S, T), torch.float32)
    if idx is not None:
        _expect("idx", idx, (B, S, L), torch.int32)
    dev = _dev(qI, qI_scale, kI, kI_scale, w, q, kv_win, kv_comp, sink, out, scores, idx)
    if scores is None:
        scores = torch.empty(B, S, T, dtype=torch.float32, device=dev)
    if idx is None:
        idx = torch.empty(B, S, L, dtype=torch.int32, device=dev)
    need = dsa_step_workspace_size(dt, B, S, H, D, T, index_topk, start_pos, W)
    workspace = _workspace(need, workspace, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_attn_step_mxfp4(_ptr(qI), _ptr(qI_scale), _ptr(kI), _ptr(kI_scale), rows, _ptr(w),
                                          float(w_scale), H_I, D_I, T, int(index_topk), int(start_pos), int(ratio),
                                          int(W), _ptr(q), ctypes.byref(win), ctypes.byref(comp), _ptr(sink),
                                          float(scale), _ptr(out), dt, B, S, H, D, _ptr(scores), _ptr(idx),
                                          _ptr(workspace), wbytes, _stream(dev, stream)))
    return out, idx, scores


def dsa_topk_workspace_size(B: int, S: int, T: int, index_topk: int) -> int:
    return int(lib.dsa_topk_workspace_size(int(B), int(S), int(T), int(index_topk)))


def dsa_step_workspace_size(dtype_code: int, B: int, S: int, H: int, D: int, T: int, index_topk: int,
                            start_pos: int, W: int) -> int:
    return int(lib.dsa_step_workspace_size(dtype_code, B, S, H, D, T, int(index_topk), int(start_pos), int(W)))


def _wbytes(workspace):
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def dsa_topk(scores, index_topk: int, start_pos: int, ratio: int, offset: int, out=None, col: int = 0,
             workspace=None, stream=None):
    """Top-k index rows; writes K = min(index_topk, T) columns of `out` [B,S,>=col+K] from `col` on."""
    dev = _dev(scores)
    _need_contig("scores", scores)
    B, S, T = scores.shape
    if scores.dtype != torch.float32:
        raise DsaError(-3, "scores must be float32")
    K = min(int(index_topk), T)
    if out is None:
        out = torch.empty(B, S, col + K, dtype=torch.int32, device=dev)
    _need_contig("idx", out)
    if out.dtype != torch.int32 or tuple(out.shape[:2]) != (B, S) or out.shape[-1] < col + K:
        raise DsaError(-2, "idx must be int32 with room for the top-k columns")
    base = ctypes.c_void_p(out.data_ptr() + 4 * col)
    workspace = _workspace(dsa_topk_workspace_size(B, S, T, index_topk), workspace, dev)
    _check(lib.dsa_topk(_ptr(scores), B, S, T, int(index_topk), int(start_pos), int(ratio), int(offset), base,
                        out.shape[-1], _ptr(workspace), _wbytes(workspace), _stream(dev, stream)))
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
    if out.dtype != torch.int32 or out.dim() != 3:
        raise DsaError(-3, "idx must be int32 [B, S, L]")
    B, S, ld = out.shape
    _check(lib.dsa_window_idx(B, S, int(start_pos), int(W), _ptr(out), ld, _stream(dev, stream)))
    return out


def dsa_select(scores, index_topk: int, start_pos: int, ratio: int, W: int, offset: int, out=None, workspace=None,
               stream=None):
    """Whole index rows [B, S, Wc + K]: window columns, then the top-k columns (one launch)."""
    B, S, T = scores.shape
    dev = _dev(scores)
    _need_contig("scores", scores)
    if scores.dtype != torch.float32:
        raise DsaError(-3, "scores must be float32")
    Wc = dsa_window_cols(S, start_pos, W)
    K = min(int(index_topk), T)
    if out is None:
        out = torch.empty(B, S, Wc + K, dtype=torch.int32, device=dev)
    _need_contig("idx", out)
    if out.dtype != torch.int32 or tuple(out.shape[:2]) != (B, S) or out.shape[-1] < Wc + K:
        raise DsaError(-2, "idx must be int32 with room for the window and top-k columns")
    workspace = _workspace(dsa_topk_workspace_size(B, S, T, index_topk), workspace, dev)
    _check(lib.dsa_select(_ptr(scores), B, S, T, int(index_topk), int(start_pos), int(ratio), int(W), int(offset),
                          _ptr(out), out.shape[-1], _ptr(workspace), _wbytes(workspace), _stream(dev, stream)))
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


def _attn_operands(q, kv_win, kv_comp, sink, comp_scales, out):
    """Shapes, dtype code, KV source descriptors and output of an attention call, checked."""
    if q.dim() != 4:
        raise DsaError(-2, "q must be [B, S, H, D]")
    _need_contig("q", q)
    B, S, H, D = q.shape
    dt = _dtype_code(q)
    if kv_win is None or kv_win.dim() != 3 or kv_win.shape[0] != B or kv_win.shape[2] != D:
        raise DsaError(-2, "kv_win must be [B, n_win, D]")
    if kv_win.dtype != q.dtype:
        raise DsaError(-3, "kv_win must have q's dtype")
    _expect("sink", sink, (H,), torch.float32)
    fp4 = kv_comp is not None and kv_comp.dtype == torch.uint8
    if kv_comp is not None:
        if kv_comp.dim() != 3 or kv_comp.shape[0] != B or kv_comp.shape[2] != (D // 2 if fp4 else D):
            raise DsaError(-2, "kv_comp must be [B, T, D] (or [B, T, D/2] uint8 fp4 nibbles)")
        if not fp4 and kv_comp.dtype != q.dtype:
            raise DsaError(-3, "kv_comp must have q's dtype (or be uint8 fp4 nibbles)")
        if fp4:
            _expect("comp_scales", comp_scales, (B, kv_comp.shape[1], D // 16), torch.uint8)
    win = kv_src(kv_win)
    comp = kv_src(kv_comp, comp_scales, DSA_KV_FP4_E4M3_G16 if fp4 else DSA_KV_DENSE)
    if out is None:
        out = torch.empty_like(q)
    _expect("o", out, q.shape, q.dtype)
    _need_contig("o", out)
    return B, S, H, D, dt, win, comp, out


def dsa_sparse_attn(q, kv_win, kv_comp, sink, idx, scale: float, comp_scales=None, out=None, workspace=None,
                    stream=None):
    """Sparse attention with a per-head sink; o [B,S,H,D] in q's dtype.

    kv_win [B, n_win, D]; kv_comp [B, T, D] in q's dtype, or [B, T, D/2] uint8 fp4 nibbles with
    comp_scales [B, T, D/16] uint8 E4M3; idx [B, S, L] int32 over [window rows | compressed rows].
    """
    B, S, H, D, dt, win, comp, out = _attn_operands(q, kv_win, kv_comp, sink, comp_scales, out)
    _need_contig("idx", idx)
    if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, S) or idx.dtype != torch.int32:
        raise DsaError(-2, "idx must be int32 [B, S, L]")
    L = idx.shape[-1]
    dev = _dev(q, kv_win, kv_comp, sink, idx, out)
    need = dsa_sparse_attn_workspace_size(dt, B, S, H, D, L)
    workspace = _workspace(need, workspace, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_attn(_ptr(q), ctypes.byref(win), ctypes.byref(comp), _ptr(sink), _ptr(idx), L,
                               float(scale), _ptr(out), dt, B, S, H, D, _ptr(workspace), wbytes,
                               _stream(dev, stream)))
    return out


def dsa_sparse_attn_rope(q, kv_win, kv_comp, sink, idx, scale: float, freqs, comp_scales=None, out=None,
                         workspace=None, stream=None):
    """dsa_sparse_attn followed by the inverse rotary embedding of o's last 2*freqs.shape[1] dims
    (freqs [S, rope_dim/2, 2] float32 cos/sin of the queries' positions), fused where the kernel can."""
    B, S, H, D, dt, win, comp, out = _attn_operands(q, kv_win, kv_comp, sink, comp_scales, out)
    _need_contig("idx", idx)
    if idx.dim() != 3 or tuple(idx.shape[:2]) != (B, S) or idx.dtype != torch.int32:
        raise DsaError(-2, "idx must be int32 [B, S, L]")
    if freqs.dim() != 3 or freqs.shape[0] != S or freqs.shape[2] != 2 or freqs.dtype != torch.float32:
        raise DsaError(-2, "freqs must be float32 [S, rope_dim/2, 2]")
    _need_contig("freqs", freqs)
    L = idx.shape[-1]
    dev = _dev(q, kv_win, kv_comp, sink, idx, out, freqs)
    workspace = _workspace(dsa_sparse_attn_workspace_size(dt, B, S, H, D, L), workspace, dev)
    _check(lib.dsa_sparse_attn_rope(_ptr(q), ctypes.byref(win), ctypes.byref(comp), _ptr(sink), _ptr(idx), L,
                                    float(scale), _ptr(out), dt, B, S, H, D, _ptr(freqs), 2 * freqs.shape[1],
                                    _ptr(workspace), _wbytes(workspace), _stream(dev, stream)))
    return out


def dsa_rope_inverse(o, freqs, stream=None):
    """In place: the inverse rotary embedding of o [B, S, H, D]'s last 2*freqs.shape[1] dims."""
    _need_contig("o", o)
    B, S, H, D = o.shape
    if freqs.dim() != 3 or freqs.shape[0] != S or freqs.dtype != torch.float32:
        raise DsaError(-2, "freqs must be float32 [S, rope_dim/2, 2]")
    _need_contig("freqs", freqs)
    dev = _dev(o, freqs)
    _check(lib.dsa_rope_inverse(_ptr(o), _dtype_code(o), B, S, H, D, _ptr(freqs), 2 * freqs.shape[1],
                                _stream(dev, stream)))
    return o


def dsa_compress_kv_write(latent, freqs, rows, scales, row0: int, stream=None):
    """Rotate, fp4-quantise and store latent [B, n, D] bf16 at rows row0.. of the fp4 cache
    (rows [B, R, D/2] uint8, scales [B, R, D/16] uint8; cache slices allowed)."""
    if latent.dtype != torch.bfloat16 or latent.dim() != 3 or latent.stride(2) != 1 or latent.stride(1) != latent.shape[2]:
        raise DsaError(-3, "latent must be bf16 [B, n, D] with dense rows")
    B, n, D = latent.shape
    if freqs.dim() != 3 or freqs.shape[0] != n or freqs.dtype != torch.float32:
        raise DsaError(-2, "freqs must be float32 [n, rope_dim/2, 2]")
    _need_contig("freqs", freqs)
    for name, t, w in (("rows", rows, D // 2), ("scales", scales, D // 16)):
        if t.dtype != torch.uint8 or t.dim() != 3 or t.shape[0] != B or t.shape[2] != w or t.stride(2) != 1 \
                or t.stride(1) != w or t.shape[1] < row0 + n:
            raise DsaError(-2, f"{name} must be uint8 [B, >= row0 + n, {w}] with dense rows")
    dev = _dev(latent, freqs, rows, scales)
    _check(lib.dsa_compress_kv_write(_ptr(latent), latent.stride(0), B, n, D, _ptr(freqs), 2 * freqs.shape[1],
                                     _ptr(rows), rows.stride(0), _ptr(scales), scales.stride(0), int(row0),
                                     _stream(dev, stream)))
    return rows, scales


def dsa_sparse_attn_select(scores, q, kv_win, kv_comp, sink, *, index_topk: int, start_pos: int, ratio: int,
                           W: int, scale: float, comp_scales=None, out=None, idx=None, workspace=None, stream=None):
    """Index rows (window + top-k, as dsa_select with offset kv_win.shape[1]) and the sparse attention
    over them; one launch for decode batches the two-phase decode kernel takes.  Returns (o, idx);
    idx [B, S, L] int32 receives the rows (allocated when not given)."""
    B, S, H, D, dt, win, comp, out = _attn_operands(q, kv_win, kv_comp, sink, comp_scales, out)
    _need_contig("scores", scores)
    T = scores.shape[-1]
    _expect("scores", scores, (B, S, T), torch.float32)
    dev = _dev(q, kv_win, kv_comp, sink, scores, out)
    Wc = dsa_window_cols(S, start_pos, W)
    L = Wc + min(int(index_topk), T)
    if idx is None:
        idx = torch.empty(B, S, L, dtype=torch.int32, device=dev)
    _need_contig("idx", idx)
    if idx.dtype != torch.int32 or tuple(idx.shape) != (B, S, L):
        raise DsaError(-2, "idx must be int32 [B, S, L] with L = window columns + top-k columns")
    need = dsa_step_workspace_size(dt, B, S, H, D, T, index_topk, start_pos, W)
    workspace = _workspace(need, workspace, dev)
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
    _need_contig("q_idx", q_idx)
    _need_contig("w", w)
    B, S, H, D, dt, win, comp, out = _attn_operands(q, kv_win, kv_comp, sink, comp_scales, out)
    if q_idx.dim() != 4 or tuple(q_idx.shape[:2]) != (B, S):
        raise DsaError(-2, "q_idx must be [B, S, H_I, D_I]")
    H_I, D_I = q_idx.shape[2], q_idx.shape[3]
    T = k_idx.shape[1]
    kbs, krs = _batched_rows("k_idx", k_idx)
    if krs != D_I:
        raise DsaError(-2, "k_idx rows must be dense")
    _expect("k_idx", k_idx, (B, T, D_I), q_idx.dtype)
    _expect("w", w, (B, S, H_I), q_idx.dtype)
    dev = _dev(q_idx, k_idx, w, q, kv_win, kv_comp, sink, out)
    Wc = dsa_window_cols(S, start_pos, W)
    L = Wc + min(int(index_topk), T)
    if scores is None:
        scores = torch.empty(B, S, T, dtype=torch.float32, device=dev)
    _expect("scores", scores, (B, S, T), torch.float32)
    _need_contig("scores", scores)
    if idx is None:
        idx = torch.empty(B, S, L, dtype=torch.int32, device=dev)
    _need_contig("idx", idx)
    if idx.dtype != torch.int32 or tuple(idx.shape) != (B, S, L):
        raise DsaError(-2, "idx must be int32 [B, S, L] with L = window columns + top-k columns")
    need = dsa_step_workspace_size(dt, B, S, H, D, T, index_topk, start_pos, W)
    workspace = _workspace(need, workspace, dev)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.dsa_sparse_attn_step(_ptr(q_idx), _ptr(k_idx), kbs, _ptr(w), float(w_scale), H_I, D_I, T,
                                    int(index_topk), int(start_pos), int(ratio), int(W), _ptr(q), ctypes.byref(win),
                                    ctypes.byref(comp), _ptr(sink), float(scale), _ptr(out), dt, B, S, H, D,
                                    _ptr(scores), _ptr(idx), _ptr(workspace), wbytes, _stream(dev, stream)))
    return out, idx, scores


def dsa_sparse_attn_step_noalloc(q_idx, k_idx, w, q, kv_win, kv_comp, sink, *, index_topk: int, start_pos: int,
                                 ratio: int, W: int, scale: float, w_scale: float, out, scores, idx,
                                 comp_scales=None, stream=None):
    """dsa_sparse_attn_step without a workspace: the library's fixed per-device scratch array is
    used (see include/dsa.h).  The caller passes every output (o, scores [B,S,T] float32, idx
    [B,S,L] int32); nothing is allocated here either."""
    _need_contig("q_idx", q_idx)
    _need_contig("w", w)
    B, S, H, D, dt, win, comp, out = _attn_operands(q, kv_win, kv_comp, sink, comp_scales, out)
    H_I, D_I = q_idx.shape[2], q_idx.shape[3]
    T = k_idx.shape[1]
    kbs, krs = _batched_rows("k_idx", k_idx)
    if krs != D_I:
        raise DsaError(-2, "k_idx rows must be dense")
    _expect("k_idx", k_idx, (B, T, D_I), q_idx.dtype)
    _expect("w", w, (B, S, H_I), q_idx.dtype)
    _expect("scores", scores, (B, S, T), torch.float32)
    L = dsa_window_cols(S, start_pos, W) + min(int(index_topk), T)
    _expect("idx", idx, (B, S, L), torch.int32)
    dev = _dev(q_idx, k_idx, w, q, kv_win, kv_comp, sink, out, scores, idx)
    _check(lib.dsa_sparse_attn_step_noalloc(_ptr(q_idx), _ptr(k_idx), kbs, _ptr(w), float(w_scale), H_I, D_I, T,
                                            int(index_topk), int(start_pos), int(ratio), int(W), _ptr(q),
                                            ctypes.byref(win), ctypes.byref(comp), _ptr(sink), float(scale),
                                            _ptr(out), dt, B, S, H, D, _ptr(scores), _ptr(idx), _stream(dev, stream)))
    return out, idx, scores


def sparse_attention_step(q, kv_win, kv_comp, qI, kI, w, sink, *, start_pos: int, ratio: int, W: int,
                          index_topk: int, scale: float, w_scale: float, comp_scales=None, index_scales=None,
                          bufs=None, stream=None):
    """One pass of the whole step: window rows, index scores, top-k, sparse attention.

    qI/kI are bf16/fp32 index rows, or uint8 MXFP4 nibbles with index_scales = (qI_scale, kI_scale).
    Returns (o, idx, scores).  `bufs` may carry preallocated 'scores', 'idx', 'o', 'workspace'.
    """
    bufs = {} if bufs is None else bufs
    B, S = q.shape[:2]
    T = kI.shape[1]
    if qI.dtype == torch.uint8:
        if index_scales is None:
            raise DsaError(-1, "MXFP4 index operands need index_scales=(qI_scale, kI_scale)")
        return dsa_sparse_attn_step_mxfp4(qI, index_scales[0], kI, index_scales[1], w, q, kv_win, kv_comp, sink,
                                          index_topk=index_topk, start_pos=start_pos, ratio=ratio, W=W, scale=scale,
                                          w_scale=w_scale, comp_scales=comp_scales, out=bufs.get("o"),
                                          scores=bufs.get("scores"), idx=bufs.get("idx"),
                                          workspace=bufs.get("workspace"), stream=stream)
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
    "dsa_init",
    "dsa_device_errors",
    "dsa_last_launches",
    "dsa_set_debug",
    "dsa_check_idx",
    "dsa_topk_plan",
    "DsaKvSrc",
    "dsa_index_scores",
    "dsa_index_scores_mxfp4",
    "dsa_index_scores_masked",
    "dsa_candidate_blocks",
    "DsaCandidates",
    "dsa_sparse_attn_step_mxfp4",
    "dsa_topk",
    "dsa_select",
    "dsa_window_cols",
    "dsa_window_idx",
    "dsa_sparse_attn",
    "dsa_sparse_attn_select",
    "dsa_sparse_attn_rope",
    "dsa_rope_inverse",
    "dsa_compress_kv_write",
    "dsa_sparse_attn_step",
    "dsa_sparse_attn_step_noalloc",
    "dsa_sparse_attn_workspace_size",
    "dsa_topk_workspace_size",
    "dsa_step_workspace_size",
    "kv_src",
    "sparse_attention_step",
    "lib",
    "ABI_VERSION",
]
