"""The allocation-free step entry point (dsa_sparse_attn_step_noalloc, through the C ABI) gives
the same bits as dsa_sparse_attn_step with a caller workspace, on two calls in a row (the second
with a smaller input), and refuses a shape whose scratch would not fit its fixed array."""
import sys

import pytest
import torch

import dsa_synth

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run_both(w, seed):
    import sparse_mqa_attention_amd as dsa

    d = dsa_synth.generate(w, seed=seed, device=DEV)
    comp = d.get("kv_comp", d.get("kv_comp_fp4"))
    kw = dict(index_topk=w.index_topk, start_pos=w.start_pos, ratio=w.ratio, W=w.W, scale=w.D ** -0.5,
              w_scale=w.D_I ** -0.5 * w.H_I ** -0.5, comp_scales=d.get("kv_comp_scale"))
    args = (d["qI"], d["kI"], d["w"], d["q"], d["kv_win"], comp, d["sink"])
    ref_o, ref_idx, ref_scores = dsa.dsa_sparse_attn_step(*args, **kw)
    ref_launches = dsa.dsa_last_launches()
    o = torch.full_like(ref_o, float("nan"))
    idx = torch.full_like(ref_idx, -7)
    scores = torch.full_like(ref_scores, float("nan"))
    dsa.dsa_sparse_attn_step_noalloc(*args, out=o, scores=scores, idx=idx, **kw)
    launches = dsa.dsa_last_launches()
    torch.cuda.synchronize()
    _log(f"  {w.name}: launches {launches} (with a workspace: {ref_launches})")
    assert launches == ref_launches
    assert torch.equal(scores, ref_scores)
    assert torch.equal(idx, ref_idx)
    assert torch.equal(o, ref_o)


def test_noalloc_step_matches_workspace_step():
    import sparse_mqa_attention_amd as dsa

    big = dsa_synth.get("decode_b32_ctx8k")
    small = dsa_synth.scaled(dsa_synth.get("decode_b32_ctx8k"), B=5, start_pos=4095, name="decode_b5_ctx4k")
    _log("no-alloc step: decode_b32_ctx8k, then a smaller decode batch")
    _run_both(big, seed=3)
    _run_both(small, seed=4)
    _log("no-alloc step: tiny prefill (no scratch needed)")
    _run_both(dsa_synth.get("tiny_prefill_f32"), seed=5)
    assert dsa.dsa_device_errors() == 0


def test_noalloc_step_refuses_oversize_shape():
    import sparse_mqa_attention_amd as dsa

    # 64 decode queries do not fit the decode kernel's resident grid; the split kernel's partials
    # (64 x 4 x 64 heads x 512 fp32) exceed the fixed scratch array
    w = dsa_synth.scaled(dsa_synth.get("decode_b32_ctx8k"), B=64, start_pos=1023, name="decode_b64_ctx1k")
    d = dsa_synth.generate(w, seed=0, device=DEV)
    o = torch.empty_like(d["q"])
    scores = torch.empty(w.B, w.S, w.T, dtype=torch.float32, device=DEV)
    idx = torch.empty(w.B, w.S, w.L, dtype=torch.int32, device=DEV)
    with pytest.raises(dsa.DsaError) as e:
        dsa.dsa_sparse_attn_step_noalloc(d["qI"], d["kI"], d["w"], d["q"], d["kv_win"], d["kv_comp"], d["sink"],
                                         index_topk=w.index_topk, start_pos=w.start_pos, ratio=w.ratio, W=w.W,
                                         scale=w.D ** -0.5, w_scale=w.D_I ** -0.5 * w.H_I ** -0.5, out=o,
                                         scores=scores, idx=idx)
    assert e.value.code == -6 and "scratch" in str(e.value)
    assert dsa.dsa_last_launches()[0] == 0
