"""The C ABI library loads, exports every entry point include/dsa.h declares, and rejects bad
arguments before anything is launched (so these run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")


def _declared():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(dsa_\w+)\s*\(", txt, flags=re.M)))


@pytest.fixture(scope="module")
def dsa():
    import sparse_mqa_attention_amd as m

    return m


def test_header_declares_the_step():
    names = _declared()
    for n in ["dsa_index_scores", "dsa_topk", "dsa_window_idx", "dsa_select", "dsa_sparse_attn",
              "dsa_sparse_attn_select", "dsa_sparse_attn_step", "dsa_last_error",
              "dsa_abi_version", "dsa_sparse_attn_workspace_size", "dsa_window_cols"]:
        assert n in names


def test_library_exports_every_declared_symbol(dsa):
    lib = ctypes.CDLL(dsa.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert dsa.lib.dsa_abi_version() == 1


def test_window_cols(dsa):
    assert dsa.dsa_window_cols(64, 0, 16) == 16
    assert dsa.dsa_window_cols(6, 0, 16) == 6
    assert dsa.dsa_window_cols(1, 8191, 128) == 128
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_window_cols(4, 10, 128)  # chunked decode is not defined by the page
    assert e.value.code == -4


def test_argument_errors_without_launch(dsa):
    lib = dsa.lib
    vp = ctypes.c_void_p
    nul = vp(0)
    # dtype
    rc = lib.dsa_index_scores(nul, nul, 0, nul, 1.0, 7, 1, 1, 1, 1, 32, 3, 1, nul, nul)
    assert rc == -3 and b"dtype" in lib.dsa_last_error()
    # T beyond what the call can see
    rc = lib.dsa_index_scores(nul, nul, 0, nul, 1.0, 1, 1, 4, 9, 4, 32, 0, 1, nul, nul)
    assert rc == -2
    # null tensors
    rc = lib.dsa_index_scores(nul, nul, 64, nul, 1.0, 1, 1, 4, 2, 4, 32, 0, 2, nul, nul)
    assert rc == -1
    # empty work is fine and launches nothing
    assert lib.dsa_index_scores(nul, nul, 0, nul, 1.0, 1, 0, 4, 2, 4, 32, 0, 2, nul, nul) == 0
    assert lib.dsa_topk(nul, 1, 1, 0, 8, 0, 4, 0, nul, 8, nul) == 0
    assert lib.dsa_topk(nul, 1, 1, 10, 8, 0, 4, 0, nul, 4, nul) == -2  # ld_idx < K
    assert lib.dsa_topk(nul, 1, 1, 10, 8, 0, 0, 0, nul, 8, nul) == -2  # ratio 0
    assert lib.dsa_topk(nul, 1, 1, 10, 8, 0, 4, 0, nul, 8, nul) == -1
    assert lib.dsa_window_idx(1, 2, 5, 4, nul, 4, nul) == -4
    assert lib.dsa_window_idx(1, 2, 0, 4, nul, 1, nul) == -2
    # whole index rows: ld_idx must hold the window and the top-k columns (2 + 8 here)
    assert lib.dsa_select(nul, 1, 2, 10, 8, 0, 4, 4, 2, nul, 9, nul) == -2
    assert lib.dsa_select(nul, 1, 2, 10, 8, 5, 4, 4, 2, nul, 10, nul) == -4  # chunked decode
    assert lib.dsa_select(nul, 1, 2, 10, 8, 0, 4, 4, 2, nul, 10, nul) == -1
    assert lib.dsa_select(nul, 0, 2, 10, 8, 0, 4, 4, 2, nul, 10, nul) == 0
    # index rows + attention: sizes, missing window source, chunked decode, empty batch, a shape
    # that needs idx (the fp32 path always runs the two calls)
    src0 = dsa.DsaKvSrc()
    src0.rows = 16
    src0.n_rows = 4
    src0.batch_stride = 4 * 64
    src0.row_stride = 64
    sel = lib.dsa_sparse_attn_select
    assert sel(vp(16), 10, 8, 0, 0, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 1, 1, 1, 1, 64, nul,
               nul, 0, nul) == -2  # ratio 0
    assert sel(vp(16), 10, 8, 0, 4, 4, vp(16), None, None, vp(16), 1.0, vp(16), 1, 1, 1, 1, 64, nul, nul, 0,
               nul) == -1
    assert sel(vp(16), 10, 8, 10, 4, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 1, 1, 4, 1, 64, nul,
               nul, 0, nul) == -4  # chunked decode
    assert sel(vp(16), 10, 8, 0, 4, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 1, 0, 1, 1, 64, nul,
               nul, 0, nul) == 0
    assert sel(vp(16), 10, 8, 0, 4, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 0, 1, 1, 1, 64, nul,
               nul, 0, nul) == -1
    # the whole step: dtype, sizes, missing window source, empty batch
    step = lib.dsa_sparse_attn_step
    common = (vp(16), vp(16), 128 * 10, vp(16), 1.0)
    assert step(*common, 32, 128, 10, 8, 0, 4, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 7, 1, 1, 1,
                64, vp(16), nul, nul, 0, nul) == -3
    assert step(*common, 32, 128, 10, 8, 0, 0, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 1, 1, 1, 1,
                64, vp(16), nul, nul, 0, nul) == -2  # ratio 0
    assert step(*common, 0, 128, 10, 8, 0, 4, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 1, 1, 1, 1,
                64, vp(16), nul, nul, 0, nul) == -2  # no index heads
    assert step(*common, 32, 128, 10, 8, 0, 4, 4, vp(16), None, None, vp(16), 1.0, vp(16), 1, 1, 1, 1, 64, vp(16),
                nul, nul, 0, nul) == -1
    assert step(*common, 32, 128, 10, 8, 0, 4, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 1, 0, 1, 1,
                64, vp(16), nul, nul, 0, nul) == 0
    # T beyond what the queries can see is the index scores' shape error
    assert step(*common, 32, 128, 10, 8, 0, 4, 4, vp(16), ctypes.byref(src0), None, vp(16), 1.0, vp(16), 1, 1, 4, 1,
                64, vp(16), nul, nul, 0, nul) == -2
    # sparse attention: unsupported head_dim, missing window source, bad format, workspace
    src = dsa.DsaKvSrc()
    src.rows = 16
    src.n_rows = 4
    src.batch_stride = 4 * 96
    src.row_stride = 96
    rc = lib.dsa_sparse_attn(vp(16), ctypes.byref(src), None, vp(16), vp(16), 4, 1.0, vp(16), 1, 1, 1, 1, 96, nul, 0,
                             nul)
    assert rc == -4
    rc = lib.dsa_sparse_attn(vp(16), None, None, vp(16), vp(16), 4, 1.0, vp(16), 1, 1, 1, 1, 64, nul, 0, nul)
    assert rc == -1
    src.row_stride = 64
    src.batch_stride = 256
    src.format = 5
    rc = lib.dsa_sparse_attn(vp(16), ctypes.byref(src), None, vp(16), vp(16), 4, 1.0, vp(16), 1, 1, 1, 1, 64, nul, 0,
                             nul)
    assert rc == -3
    src.format = 0
    need = lib.dsa_sparse_attn_workspace_size(1, 2, 1, 64, 512, 640)
    assert need > 0  # two decode queries split their index rows over several workgroups
    rc = lib.dsa_sparse_attn(vp(16), ctypes.byref(src), None, vp(16), vp(16), 640, 1.0, vp(16), 1, 2, 1, 64, 64, nul,
                             0, nul)
    assert rc == -6
    assert lib.dsa_sparse_attn_workspace_size(1, 1, 8192, 64, 512, 640) == 0  # prefill fills the GPU unsplit
    # fp4 rows need bf16 and scales
    src2 = dsa.DsaKvSrc()
    src2.rows = 16
    src2.n_rows = 2
    src2.batch_stride = 64
    src2.row_stride = 32
    src2.format = 1
    rc = lib.dsa_sparse_attn(vp(16), ctypes.byref(src), ctypes.byref(src2), vp(16), vp(16), 4, 1.0, vp(16), 1, 1, 1,
                             1, 64, nul, 0, nul)
    assert rc == -1  # scales NULL


def test_no_cpu_fallback_in_binding():
    # the product package never imports the oracle
    src = open(os.path.join(ROOT, "sparse_mqa_attention_amd", "__init__.py")).read()
    assert "oracle" not in src.replace("oracle is", "")
