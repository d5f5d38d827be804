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
              "dsa_abi_version", "dsa_sparse_attn_workspace_size", "dsa_window_cols", "dsa_init",
              "dsa_device_errors", "dsa_last_launch_count", "dsa_last_launches", "dsa_set_debug", "dsa_check_idx",
              "dsa_topk_plan", "dsa_topk_workspace_size", "dsa_step_workspace_size", "dsa_index_scores_mxfp4",
              "dsa_sparse_attn_step_mxfp4", "dsa_sparse_attn_step_noalloc"]:
        assert n in names


def test_library_exports_every_declared_symbol(dsa):
    lib = ctypes.CDLL(dsa.LIB_PATH)
    for n in _declared():
        assert hasattr(lib, n), n
    assert dsa.lib.dsa_abi_version() == 2


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
    assert lib.dsa_topk(nul, 1, 1, 0, 8, 0, 4, 0, nul, 8, nul, 0, nul) == 0
    assert lib.dsa_topk(nul, 1, 1, 10, 8, 0, 4, 0, nul, 4, nul, 0, nul) == -2  # ld_idx < K
    assert lib.dsa_topk(nul, 1, 1, 10, 8, 0, 0, 0, nul, 8, nul, 0, nul) == -2  # ratio 0
    assert lib.dsa_topk(nul, 1, 1, 10, 8, 0, 4, 0, nul, 8, nul, 0, nul) == -1
    assert lib.dsa_window_idx(1, 2, 5, 4, nul, 4, nul) == -4
    assert lib.dsa_window_idx(1, 2, 0, 4, nul, 1, nul) == -2
    # whole index rows: ld_idx must hold the window and the top-k columns (2 + 8 here)
    assert lib.dsa_select(nul, 1, 2, 10, 8, 0, 4, 4, 2, nul, 9, nul, 0, nul) == -2
    assert lib.dsa_select(nul, 1, 2, 10, 8, 5, 4, 4, 2, nul, 10, nul, 0, nul) == -4  # chunked decode
    assert lib.dsa_select(nul, 1, 2, 10, 8, 0, 4, 4, 2, nul, 10, nul, 0, nul) == -1
    assert lib.dsa_select(nul, 0, 2, 10, 8, 0, 4, 4, 2, nul, 10, nul, 0, nul) == 0
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


def test_workspace_has_header(dsa):
    lib = dsa.lib
    # every nonzero workspace starts with the 4 KiB counter header
    need = lib.dsa_sparse_attn_workspace_size(1, 32, 1, 64, 512, 640)
    assert need > 4096
    split = lib.dsa_sparse_attn_workspace_size(1, 2, 3, 32, 128, 130)  # general kernel's partials
    assert split > 4096


def test_check_idx_host(dsa):
    """The DSA_DEBUG range check (host side): -1 and [0, rows) pass, anything else is rejected
    with the first bad position."""
    import numpy as np

    assert dsa.dsa_check_idx(np.array([-1, 0, 5, 9], dtype=np.int32), 10) == (True, -1)
    assert dsa.dsa_check_idx(np.array([3, -1, 10, 11], dtype=np.int32), 10) == (False, 2)
    assert dsa.dsa_check_idx(np.array([0, -2], dtype=np.int32), 10) == (False, 1)
    assert dsa.dsa_check_idx(np.zeros(0, dtype=np.int32), 0) == (True, -1)
    assert dsa.dsa_check_idx(np.array([0], dtype=np.int32), 0) == (False, 0)
    big = np.full(1 << 16, 7, dtype=np.int32)
    big[-1] = -3
    assert dsa.dsa_check_idx(big, 8) == (False, (1 << 16) - 1)
    prev = dsa.dsa_set_debug(True)
    assert dsa.dsa_set_debug(prev) is True


@pytest.mark.parametrize("rows,T", [(1024, 1), (1500, 1), (2047, 1), (2047, 2), (1024, 3), (1100, 4000), (5000, 64),
                                    (4096, 2048), (2048, 8192), (3000, 9000), (1023, 5)])
def test_topk_row_split(dsa, rows, T):
    """The one-wave top-k kernel reads a whole number of 64-key groups per row (up to 64*KPL keys):
    every row it gets must keep that span inside the B*S*T scores, and the rest go to the per-row
    kernel, never a negative count."""
    wave, block = dsa.dsa_topk_plan(1, rows, T)
    assert wave >= 0 and block >= 0 and wave + block == rows
    if rows < 1024 or T > 8192:
        assert wave == 0
        return
    kpl = 32 if T <= 2048 else 64 if T <= 4096 else 128
    if wave:
        assert (wave - 1) * T + 64 * kpl <= rows * T  # the last wave row's reads stay in the buffer
    if block and wave + 1 <= rows - 1:
        assert wave * T + 64 * kpl > rows * T  # the split point is the first row that would overrun


def test_binding_validates_before_launch(dsa):
    """Mis-shaped or mistyped operands are refused by the binding with DSA_ERR_SHAPE/DTYPE before
    any pointer reaches the library (CPU tensors: the checks run ahead of the device check)."""
    import torch

    q = torch.zeros(1, 2, 4, 64, dtype=torch.bfloat16)
    kv = torch.zeros(1, 5, 64, dtype=torch.bfloat16)
    idx = torch.zeros(1, 2, 3, dtype=torch.int32)
    sink = torch.zeros(4)
    cases = [
        (dict(sink=torch.zeros(4, dtype=torch.bfloat16)), -3),  # sink must be float32
        (dict(sink=torch.zeros(5)), -2),                        # sink must be [H]
        (dict(kv_win=torch.zeros(1, 5, 64)), -3),              # kv dtype differs from q
        (dict(kv_win=torch.zeros(1, 5, 32, dtype=torch.bfloat16)), -2),
        (dict(out=torch.zeros(1, 2, 4, 32, dtype=torch.bfloat16)), -2),
        (dict(idx=torch.zeros(1, 2, 3, dtype=torch.int64)), -2),
        (dict(kv_comp=torch.zeros(1, 3, 64)), -3),
    ]
    for over, code in cases:
        a = dict(q=q, kv_win=kv, kv_comp=None, sink=sink, idx=idx, out=None)
        a.update(over)
        with pytest.raises(dsa.DsaError) as e:
            dsa.dsa_sparse_attn(a["q"], a["kv_win"], a["kv_comp"], a["sink"], a["idx"], 1.0, out=a["out"])
        assert e.value.code == code, (over, e.value)
    qI = torch.zeros(1, 2, 4, 32, dtype=torch.bfloat16)
    kI = torch.zeros(1, 3, 32, dtype=torch.bfloat16)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_index_scores(qI, kI, torch.zeros(1, 2, 4), 1.0, 0, 1)  # w dtype differs
    assert e.value.code == -3
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_index_scores(qI, kI, torch.zeros(1, 2, 4, dtype=torch.bfloat16), 1.0, 0, 1,
                             out=torch.zeros(1, 2, 4))
    assert e.value.code == -2
    # the whole step: scores of the wrong shape
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_sparse_attn_step(qI, kI, torch.zeros(1, 2, 4, dtype=torch.bfloat16), q, kv, None, sink, index_topk=2,
                                 start_pos=0, ratio=1, W=2, scale=1.0, w_scale=1.0, scores=torch.zeros(1, 2, 5))
    assert e.value.code == -2


def test_init_and_errors_need_a_device(dsa):
    """Without a GPU, the set-up and error-flag calls fail cleanly with an error code."""
    import ctypes

    import torch

    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert dsa.lib.dsa_init(0) == -5
    v = ctypes.c_uint32(7)
    assert dsa.lib.dsa_device_errors(0, ctypes.byref(v)) == -5
    assert dsa.lib.dsa_device_errors(0, None) == -1
    assert dsa.lib.dsa_init(-1) == -2


def test_workspace_sizes(dsa):
    """Long rows of few queries get the split select's candidate space; many rows (prefill) and
    short rows none; the step's size covers both the selection and the attention."""
    assert dsa.dsa_topk_workspace_size(16, 1, 65536, 512) == 4096 + 16 * 16 * 512 * 8
    assert dsa.dsa_topk_workspace_size(16, 1, 16384, 512) == 0     # one workgroup per row is as fast
    assert dsa.dsa_topk_workspace_size(16, 1, 16385, 512) == 4096 + 16 * 5 * 512 * 8
    assert dsa.dsa_topk_workspace_size(32, 1, 2048, 512) == 0       # short rows: one workgroup each
    assert dsa.dsa_topk_workspace_size(1, 8192, 8192, 512) == 0     # many rows: one wave each
    assert dsa.dsa_topk_workspace_size(1, 1, 65536, 8192) == 0      # candidates beyond one merge
    for args in [(1, 16, 1, 64, 512, 65536, 512, 65535, 128), (1, 32, 1, 64, 512, 2048, 512, 8191, 128),
                 (1, 1, 8192, 64, 512, 2048, 512, 0, 128)]:
        dt, B, S, H, D, T, K, sp, W = args
        step = dsa.dsa_step_workspace_size(*args)
        L = dsa.dsa_window_cols(S, sp, W) + min(K, T)
        assert step >= dsa.dsa_sparse_attn_workspace_size(dt, B, S, H, D, L)
        assert step >= dsa.dsa_topk_workspace_size(B, S, T, K)
