"""GPU parity of the HIP path (through the C ABI) against the CPU oracle.

Inputs come from the seeded generator; expected values from the oracle only.  Sizes span
several tiles with ragged tails; the full-size workloads are checked in full where the oracle
finishes in seconds (tiny prefill, both decode workloads) and on sampled queries otherwise.
"""
import math
import sys

import numpy as np
import pytest
import torch

import dsa_synth
import oracle
from parity import ATTN_TOL, check_topk_row, max_abs_err, sample_rows, score_bound

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _dsa():
    import sparse_mqa_attention_amd as dsa

    return dsa


def _log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _to_dev(d):
    return {k: v.to(DEV) for k, v in d.items()}


def _launched():
    """(count, names) of the kernels the last library call on this thread launched."""
    return _dsa().dsa_last_launches()


def _assert_one_launch(kind):
    n, names = _launched()
    assert n == 1 and kind in names, f"expected one {kind} launch, got {n}: {names}"


def _kv_cat64(cpu_inputs, w):
    if w.comp_fmt == "fp4":
        comp = oracle.fp4_rows_decode(cpu_inputs["kv_comp_fp4"], cpu_inputs["kv_comp_scale"])
    else:
        comp = cpu_inputs["kv_comp"]
    return oracle.kv_concat(cpu_inputs["kv_win"], comp)


# ------------------------------------------------------------------------ window rows
@pytest.mark.parametrize("B,S,sp,W", [(2, 6, 0, 4), (1, 300, 0, 128), (3, 1, 2, 4), (2, 1, 9, 4), (4, 1, 8191, 128),
                                      (1, 1, 65535, 128), (1, 64, 0, 16), (2, 1, 127, 128)])
def test_window_idx(B, S, sp, W):
    dsa = _dsa()
    Wc = dsa.dsa_window_cols(S, sp, W)
    out = torch.full((B, S, Wc + 3), 77, dtype=torch.int32, device=DEV)
    dsa.dsa_window_idx(out, sp, W)
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got[..., :Wc], oracle.window_rows(W, B, S, sp))
    assert np.all(got[..., Wc:] == 77)  # columns past the window untouched


# ------------------------------------------------------------------------ top-k (integer work: bit-exact)
@pytest.mark.parametrize("B,S,T,K,sp,ratio,kind", [
    (1, 64, 16, 8, 0, 4, "ties"),
    (2, 37, 100, 8, 0, 2, "normal"),
    (1, 700, 300, 64, 0, 1, "ties"),
    (2, 1, 1000, 512, 3999, 4, "normal"),
    (1, 1, 2048, 512, 8191, 4, "zeros"),
    (1, 3000, 2048, 512, 0, 4, "normal"),
    (3, 1, 4000, 512, 15999, 4, "ties"),
    (1, 1, 5000, 512, 19999, 4, "normal"),
    (2, 1, 16384, 512, 65535, 4, "normal"),
    (1, 1, 16384, 512, 65535, 4, "ties"),
    (1, 1, 30000, 700, 29999, 1, "normal"),
    # the page config's ratio 1 at 64K context: 65536 scores per row (keys re-read per pass)
    (2, 1, 65536, 512, 65535, 1, "normal"),
    (1, 1, 65536, 512, 65535, 1, "ties"),
    (3, 1, 40000, 512, 79999, 2, "zeros"),
    # split select: a chunk boundary inside the visible part, K beyond a chunk's visible count
    (4, 1, 20000, 512, 20000, 1, "ties"),
    (2, 1, 17000, 4000, 16999, 1, "normal"),
    (3, 2, 24000, 700, 47998, 2, "normal"),
    (1, 3, 600, 1, 1797, 3, "normal"),
    # 1024+ rows: one wave per row (2048, 4096 and 8192 keys per lane group)
    (1, 1100, 4000, 512, 0, 1, "ties"),
    (2, 600, 8000, 300, 100, 2, "normal"),
    (1, 1030, 8192, 512, 0, 4, "zeros"),
    (1, 1500, 1999, 7, 0, 1, "ties"),
    # tiny T at 1024..2047 rows: most rows' one-wave reads would pass the end of the scores, so
    # they go to the per-row kernel
    (1, 1500, 1, 1, 0, 1, "normal"),
    (1, 2047, 1, 4, 0, 1, "normal"),
    (1, 1024, 2, 1, 0, 1, "ties"),
    (3, 700, 2, 2, 0, 1, "normal"),
])
def test_topk_bit_exact(B, S, T, K, sp, ratio, kind):
    """Given the same float32 scores, the GPU selection equals the oracle's exactly."""
    dsa = _dsa()
    _log(f"topk case B={B} S={S} T={T} K={K} sp={sp} r={ratio} {kind}")
    rng = np.random.default_rng(T + K + S)
    if kind == "ties":
        s = rng.integers(-4, 5, size=(B, S, T)).astype(np.float32)
    elif kind == "zeros":
        s = rng.integers(0, 2, size=(B, S, T)).astype(np.float32) * rng.choice([-1.0, 1.0], size=(B, S, T)).astype(
            np.float32) * 0.0
        s[..., ::7] = rng.standard_normal(s[..., ::7].shape).astype(np.float32)
    else:
        s = rng.standard_normal((B, S, T)).astype(np.float32)
    c = oracle.visible_count(np.arange(S), sp, ratio)
    s[:, np.arange(T)[None, :] >= np.minimum(c, T)[:, None]] = -np.inf
    scores = torch.from_numpy(s).to(DEV)
    off = 5
    Kk = min(K, T)
    exp = oracle.topk_select(s.astype(np.float64), K, sp, ratio, off)
    out = torch.full((B, S, 2 + Kk), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_topk(scores, K, sp, ratio, off, out=out, col=2)
    names = _launched()[1]
    split = dsa.dsa_topk_workspace_size(B, S, T, K) > 0
    assert ("topk_split_chunk" in names) == split, names
    got = out.cpu().numpy()
    assert np.all(got[..., :2] == -7)
    np.testing.assert_array_equal(got[..., 2:], exp)
    if split:  # the same rows without a workspace: one workgroup per row
        out2 = torch.full((B, S, Kk), -7, dtype=torch.int32, device=DEV)
        rc = dsa.lib.dsa_topk(dsa._ptr(scores), B, S, T, K, sp, ratio, off, dsa._ptr(out2), Kk, None, 0,
                              dsa._stream(scores.device, None))
        assert rc == 0 and "topk_block" in _launched()[1]
        np.testing.assert_array_equal(out2.cpu().numpy(), exp)


@pytest.mark.parametrize("B,S,T,K,sp,ratio,W", [
    (1, 64, 16, 8, 0, 4, 16),        # prefill, window narrower than the chunk
    (2, 37, 100, 8, 0, 2, 128),      # prefill, window wider than the chunk
    (4, 1, 2048, 512, 8191, 4, 128),  # decode
    (2, 1, 300, 512, 1199, 4, 128),  # decode, fewer rows than index_topk
    (1, 1100, 4000, 512, 0, 1, 128),  # one wave per row, tail rows on the per-row kernel
    (3, 1, 0, 512, 2, 4, 4),         # nothing compressed yet: window part only
])
def test_select_whole_rows(B, S, T, K, sp, ratio, W):
    """One call writes each index row: the window part, then the top-k part, exactly as the oracle."""
    dsa = _dsa()
    _log(f"select case B={B} S={S} T={T} K={K} sp={sp} r={ratio} W={W}")
    rng = np.random.default_rng(7 * T + K + S)
    s = rng.standard_normal((B, S, max(T, 1))).astype(np.float32)[..., :T]
    c = oracle.visible_count(np.arange(S), sp, ratio)
    s[:, np.arange(T)[None, :] >= np.minimum(c, T)[:, None]] = -np.inf
    scores = torch.from_numpy(np.ascontiguousarray(s)).to(DEV)
    Wc = dsa.dsa_window_cols(S, sp, W)
    Kk = min(K, T)
    out = torch.full((B, S, Wc + Kk + 1), -7, dtype=torch.int32, device=DEV)
    dsa.dsa_select(scores, K, sp, ratio, W, W, out=out)
    got = out.cpu().numpy()
    np.testing.assert_array_equal(got[..., :Wc], oracle.window_rows(W, B, S, sp))
    if Kk:
        np.testing.assert_array_equal(got[..., Wc:Wc + Kk], oracle.topk_select(s.astype(np.float64), K, sp, ratio, W))
    assert np.all(got[..., Wc + Kk:] == -7)  # columns past the row untouched


# ------------------------------------------------------------------------ index scores
def _check_scores(got, qI, kI, w, w_scale, sp, ratio, rows=None, ctx=""):
    q64 = qI.float().numpy().astype(np.float64)
    k64 = kI.float().numpy().astype(np.float64)
    w64 = w.float().numpy().astype(np.float64)
    if rows is None:
        exp = oracle.index_scores(q64, k64, w64, w_scale, sp, ratio)
        B, S = exp.shape[:2]
        rows = [(b, t) for b in range(B) for t in range(S)]
        exp_rows = exp.reshape(B * S, -1)
    else:
        exp_rows = oracle.index_scores_rows(q64, k64, w64, w_scale, sp, ratio, rows)
    worst = 0.0
    for n, (b, t) in enumerate(rows):
        g = got[b, t]
        e = exp_rows[n]
        inv = np.isinf(e)
        assert np.all(np.isneginf(g[inv])), f"{ctx} ({b},{t}): masked entries must be -inf"
        bound = score_bound(q64[b, t][None], k64[b], w64[b, t][None], w_scale)[0]
        err = np.abs(g[~inv] - e[~inv])
        lim = 1e-5 * bound[~inv] + 1e-30
        assert np.all(err <= lim), f"{ctx} ({b},{t}): score error {err.max():.3e} above the fp32 bound"
        if err.size:
            worst = max(worst, float((err / lim).max()))
    return worst


@pytest.mark.parametrize("B,S,sp,T,H,DI,ratio,dtype", [
    (1, 64, 0, 16, 4, 32, 4, "f32"),
    (2, 70, 0, 35, 32, 128, 2, "bf16"),
    (1, 300, 0, 300, 4, 32, 1, "bf16"),
    (2, 33, 0, 16, 48, 64, 2, "bf16"),
    (3, 1, 1234, 308, 32, 128, 4, "bf16"),
    (1, 9, 0, 2, 16, 256, 4, "bf16"),
    (2, 17, 40, 28, 32, 128, 2, "bf16"),
    # 64+ queries at index head dim 128: the key-streaming prefill kernel
    (1, 200, 37, 130, 20, 128, 1, "bf16"),
    (2, 96, 0, 24, 32, 128, 4, "bf16"),
    (1, 130, 5, 1, 32, 128, 4, "bf16"),
    (1, 520, 0, 260, 32, 128, 2, "bf16"),
])
def test_index_scores_small(B, S, sp, T, H, DI, ratio, dtype):
    dsa = _dsa()
    _log(f"index_scores case B={B} S={S} sp={sp} T={T} H={H} DI={DI} r={ratio} {dtype}")
    g = torch.Generator().manual_seed(S * 7 + T)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    qI = torch.randn(B, S, H, DI, generator=g).to(dt)
    kI = torch.randn(B, T + 3, DI, generator=g).to(dt)[:, :T]  # batch stride larger than T*DI
    w = (torch.randn(B, S, H, generator=g) * 0.5).to(dt)
    w_scale = DI ** -0.5 * H ** -0.5
    got = dsa.dsa_index_scores(qI.to(DEV), kI.to(DEV), w.to(DEV), w_scale, sp, ratio).cpu().numpy()
    _check_scores(got, qI, kI.contiguous(), w, w_scale, sp, ratio, ctx="small")


# ------------------------------------------------------------------------ sparse attention
def _rand_idx(rng, B, S, L, n, frac_invalid=0.15):
    idx = rng.integers(0, n, size=(B, S, L))
    idx[rng.random((B, S, L)) < frac_invalid] = -1
    return idx.astype(np.int32)


@pytest.mark.parametrize("B,S,H,D,nw,nc,L,dtype,fp4", [
    (1, 5, 4, 64, 20, 16, 24, "f32", False),
    (2, 3, 16, 64, 40, 30, 77, "bf16", False),
    (1, 2, 32, 128, 33, 100, 130, "bf16", False),
    (2, 2, 48, 256, 64, 64, 96, "bf16", False),
    (1, 3, 64, 512, 128, 500, 640, "bf16", False),
    (3, 1, 64, 512, 128, 2048, 640, "bf16", False),
    (1, 300, 64, 512, 300, 75, 200, "bf16", False),
    (2, 2, 64, 512, 128, 256, 300, "bf16", True),
    (1, 260, 64, 512, 260, 65, 100, "bf16", True),
    (2, 2, 100, 128, 16, 16, 40, "bf16", False),
    (1, 2, 8, 512, 16, 16, 33, "bf16", False),
    # many queries at head_dim 512: the one-workgroup-per-query prefill kernel
    (2, 160, 64, 512, 160, 300, 1024, "bf16", False),
    (1, 256, 40, 512, 256, 100, 77, "bf16", True),
    (1, 264, 16, 512, 264, 50, 33, "bf16", False),
    (1, 256, 64, 512, 256, 1000, 1025, "bf16", False),
    (1, 288, 40, 512, 288, 90, 70, "bf16", False),  # heads 32..39: a wave with 8 of its 32 heads
    # 1024+ queries, a count no workgroup size divides
    (1, 1027, 64, 512, 1027, 80, 160, "bf16", False),
    (1, 1030, 40, 512, 1030, 60, 70, "bf16", True),
])
def test_sparse_attn(B, S, H, D, nw, nc, L, dtype, fp4):
    dsa = _dsa()
    _log(f"sparse_attn case B={B} S={S} H={H} D={D} nw={nw} nc={nc} L={L} {dtype} fp4={fp4}")
    g = torch.Generator().manual_seed(B * 1000 + S * 10 + H + D)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.randn(B, S, H, D, generator=g).to(dt)
    kv_win = torch.randn(B, nw, D, generator=g).to(dt)
    sink = torch.randn(H, generator=g)
    if fp4:
        packed, scales = dsa_synth.encode_fp4_e2m1_e4m3(torch.randn(B, nc, D, generator=g), 16)
        comp64 = oracle.fp4_rows_decode(packed, scales)
        comp_dev, sc_dev = packed.to(DEV), scales.to(DEV)
    else:
        comp = torch.randn(B, nc, D, generator=g).to(dt)
        comp64, comp_dev, sc_dev = comp, comp.to(DEV), None
    rng = np.random.default_rng(L)
    idx = _rand_idx(rng, B, S, L, nw + nc)
    idx[0, 0, :] = -1  # a query with no valid slot
    if L >= 96:
        idx[0, min(1, S - 1), 32:64] = -1  # a whole 32-slot tile without a valid slot
    if L > 3:
        idx[-1, -1, 1] = idx[-1, -1, 0] = max(idx[-1, -1, 0], 0)  # a duplicate
    scale = D ** -0.5
    o = dsa.dsa_sparse_attn(q.to(DEV), kv_win.to(DEV), comp_dev, sink.to(DEV), torch.from_numpy(idx).to(DEV), scale,
                            comp_scales=sc_dev)
    kv = oracle.kv_concat(kv_win, comp64)
    exp = oracle.sparse_attn(q, kv, sink, idx, scale)
    got = o.float().cpu().numpy()
    err = max_abs_err(got, exp)
    _log(f"  max abs err {err:.3e}")
    assert np.all(got[0, 0] == 0)
    assert err <= ATTN_TOL[dtype], err


# ------------------------------------------------------------------------ whole step per workload
def _step(w, dev_in, bufs=None):
    dsa = _dsa()
    mx = "qI_fp4" in dev_in
    return dsa.sparse_attention_step(
        dev_in["q"], dev_in["kv_win"], dev_in.get("kv_comp", dev_in.get("kv_comp_fp4")),
        dev_in["qI_fp4"] if mx else dev_in["qI"], dev_in["kI_fp4"] if mx else dev_in["kI"],
        dev_in["w"], dev_in["sink"], start_pos=w.start_pos, ratio=w.ratio, W=w.W, index_topk=w.index_topk,
        scale=w.D ** -0.5, w_scale=w.D_I ** -0.5 * w.H_I ** -0.5, comp_scales=dev_in.get("kv_comp_scale"),
        index_scales=(dev_in["qI_scale"], dev_in["kI_scale"]) if mx else None, bufs=bufs)


def _index_f64(cpu_in):
    """Index queries and keys as float64 arrays (the MXFP4 ones decoded by the oracle)."""
    if "qI_fp4" in cpu_in:
        return (oracle.mxfp4_rows_decode(cpu_in["qI_fp4"], cpu_in["qI_scale"]),
                oracle.mxfp4_rows_decode(cpu_in["kI_fp4"], cpu_in["kI_scale"]))
    return (cpu_in["qI"].float().numpy().astype(np.float64), cpu_in["kI"].float().numpy().astype(np.float64))


def _check_step(w, cpu_in, o, idx, scores, rows):
    """Scores within the fp32 bound, window rows exact, top-k by the parity rules, and the
    attention output against the oracle on the GPU's own index rows."""
    w_scale = w.D_I ** -0.5 * w.H_I ** -0.5
    got_scores = {}
    sc = scores.cpu() if scores is not None else None
    for (b, t) in rows:
        got_scores[(b, t)] = sc[b, t].numpy() if sc is not None else None
    q64, k64 = _index_f64(cpu_in)
    w64 = cpu_in["w"].float().numpy().astype(np.float64)
    exp_rows = oracle.index_scores_rows(q64, k64, w64, w_scale, w.start_pos, w.ratio, rows)
    idx_cpu = idx.cpu().numpy()
    win = oracle.window_rows(w.W, w.B, w.S, w.start_pos)
    rules = {}
    for n, (b, t) in enumerate(rows):
        e = exp_rows[n]
        g = got_scores[(b, t)]
        inv = np.isinf(e)
        assert np.all(np.isneginf(g[inv]))
        bound = score_bound(q64[b, t][None], k64[b], w64[b, t][None], w_scale)[0]
        assert np.all(np.abs(g[~inv] - e[~inv]) <= 1e-5 * bound[~inv] + 1e-30), (b, t)
        np.testing.assert_array_equal(idx_cpu[b, t, :w.Wc], win[b, t])
        c = int(min(w.T, oracle.visible_count(t, w.start_pos, w.ratio)))
        rule = check_topk_row(idx_cpu[b, t, w.Wc:], e, w.K, c, w.n_win, ctx=f"{w.name} ({b},{t})")
        rules[rule] = rules.get(rule, 0) + 1
    kv = _kv_cat64(cpu_in, w)
    exp_o = oracle.sparse_attn_rows(cpu_in["q"], kv, cpu_in["sink"], idx_cpu, w.D ** -0.5, rows)
    got_o = np.stack([o[b, t].float().cpu().numpy() for (b, t) in rows])
    err = max_abs_err(got_o, exp_o)
    _log(f"  {w.name}: {len(rows)} rows, top-k rules {rules}, attention max abs err {err:.3e}")
    assert err <= ATTN_TOL[w.dtype], err
    return err


@pytest.mark.parametrize("name", ["tiny_prefill_f32", "decode_b32_ctx8k", "decode_b16_ctx64k"])
def test_step_full(name):
    w = dsa_synth.get(name)
    _log(f"step {name} (full check)")
    cpu_in = dsa_synth.generate(w, seed=0)
    dev_in = _to_dev(cpu_in)
    o, idx, scores = _step(w, dev_in)
    n, names = _launched()
    _log(f"  launches: {n} {names}")
    if name == "decode_b32_ctx8k":
        _assert_one_launch("score+select")  # the launch configuration the benchmark times
    torch.cuda.synchronize()
    rows = [(b, t) for b in range(w.B) for t in range(w.S)]
    _check_step(w, cpu_in, o, idx, scores, rows)
    assert _dsa().dsa_device_errors() == 0


@pytest.mark.parametrize("name,S", [("prefill_s8k", 640), ("prefill_s32k_fp4", 700), ("prefill_s8k", 2100)])
def test_step_reduced_prefill(name, S):
    """Prefill workloads cut to S queries (several tiles and the c(t) = K crossover when S > 2048)."""
    w = dsa_synth.scaled(dsa_synth.get(name), S=S, name=f"{name}_S{S}")
    _log(f"step {w.name}")
    cpu_in = dsa_synth.generate(w, seed=0)
    dev_in = _to_dev(cpu_in)
    o, idx, scores = _step(w, dev_in)
    torch.cuda.synchronize()
    rows = sample_rows(w, n_random=24)
    rows = sorted(set(rows + [(0, t) for t in range(0, w.S, max(1, w.S // 48))]))
    _check_step(w, cpu_in, o, idx, scores, rows)


@pytest.mark.parametrize("name", ["prefill_s8k", "prefill_s32k_fp4"])
def test_step_full_size_sampled(name):
    """The full prefill workloads, in the launch configuration the benchmark times, on sampled queries."""
    w = dsa_synth.get(name)
    _log(f"step {name} (full size, sampled)")
    dev_in = dsa_synth.generate(w, seed=0, device=DEV)
    o, idx, scores = _step(w, dev_in)
    torch.cuda.synchronize()
    rows = sample_rows(w, n_random=10)
    need = {"q", "kv_win", "kv_comp", "kv_comp_fp4", "kv_comp_scale", "kI", "sink"}
    cpu_in = {k: v.cpu() for k, v in dev_in.items() if k in need}
    # only the sampled queries' index q/weights are needed on the host
    cpu_in["qI"] = dev_in["qI"].cpu()
    cpu_in["w"] = dev_in["w"].cpu()
    _check_step(w, cpu_in, o, idx, scores, rows)
    # every query with no visible compressed row attends to its window only; c(t) <= K rows are exact
    idx_cpu = idx[0, : min(w.S, 4 * w.K)].cpu().numpy()
    c = oracle.visible_count(np.arange(idx_cpu.shape[0]), 0, w.ratio)
    for t in range(0, idx_cpu.shape[0], 97):
        n = int(min(w.K, c[t]))
        np.testing.assert_array_equal(idx_cpu[t, w.Wc:w.Wc + n], w.n_win + np.arange(n) if c[t] <= w.K else
                                      idx_cpu[t, w.Wc:w.Wc + n])
        assert np.all(idx_cpu[t, w.Wc + n:] == -1)


# ------------------------------------------------------------------------ index rows + attention in one call
@pytest.mark.parametrize("B,T,ctx,kind", [
    (32, 2048, 8192, "normal"),  # decode, one launch: every workgroup selects its query's row
    (5, 1999, 7996, "ties"),     # 16 splits, ties at the threshold go to the lower rows
    (3, 300, 1200, "normal"),    # fewer visible rows than index_topk: all kept, -1 tail
    (4, 4000, 16000, "normal"),  # more than 2048 scores per row: the select and attention calls
])
def test_sparse_attn_select(B, T, ctx, kind):
    """The index rows written out equal the oracle's window + top-k rows exactly, and the output
    matches the oracle's attention over those rows; two calls in a row."""
    dsa = _dsa()
    _log(f"select+attn case B={B} T={T} ctx={ctx} {kind}")
    H, D, nw, K, ratio, S = 64, 512, 128, 512, 4, 1
    sp = ctx - 1
    g = torch.Generator().manual_seed(B * 7 + T)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    kv_win = torch.randn(B, nw, D, generator=g).to(torch.bfloat16)
    kv_comp = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    rng = np.random.default_rng(T + B)
    if kind == "ties":
        sc = rng.integers(-4, 5, size=(B, S, T)).astype(np.float32)
    else:
        sc = rng.standard_normal((B, S, T)).astype(np.float32)
    c = oracle.visible_count(np.arange(S), sp, ratio)
    sc[:, np.arange(T)[None, :] >= np.minimum(c, T)[:, None]] = -np.inf
    exp_idx = np.concatenate([oracle.window_rows(nw, B, S, sp), oracle.topk_select(sc.astype(np.float64), K, sp,
                                                                                   ratio, nw)], axis=-1)
    scale = D ** -0.5
    exp_o = oracle.sparse_attn(q, oracle.kv_concat(kv_win, kv_comp), sink, exp_idx, scale)
    args = (torch.from_numpy(sc).to(DEV), q.to(DEV), kv_win.to(DEV), kv_comp.to(DEV), sink.to(DEV))
    for call in range(2):
        o, idx = dsa.dsa_sparse_attn_select(*args, index_topk=K, start_pos=sp, ratio=ratio, W=nw, scale=scale)
        n, names = _launched()
        _log(f"  launches: {n} {names}")
        if T <= 2048:
            _assert_one_launch("select")
        else:
            assert n >= 2 and "sparse_attn_decode<" in names, names
        np.testing.assert_array_equal(idx.cpu().numpy(), exp_idx)
        err = max_abs_err(o.float().cpu().numpy(), exp_o)
        _log(f"  call {call}: max abs err {err:.3e}")
        assert err <= ATTN_TOL["bf16"], err


# ------------------------------------------------------------------------ the whole step in one call
@pytest.mark.parametrize("B,T,ctx,H_I", [
    (32, 2048, 8192, 32),   # decode, one launch: 8 workgroups per query score 256 rows each
    (5, 1999, 7996, 64),    # 16 workgroups per query, two MFMA tiles of index heads, ragged tail;
                            # the grid is padded to 8 queries
    (3, 300, 1200, 40),     # fewer visible rows than index_topk: all kept, -1 tail
    (16, 100, 400, 8),      # most workgroups score no rows; score rows share cache lines
    (8, 1000, 4000, 64),    # 16 workgroups per query, 64 index heads
    (24, 777, 3108, 40),    # 8 workgroups per query, 40 index heads, ragged T
    (4, 4000, 16000, 32),   # more than 2048 scores per row: index scores, then the select call
])
def test_sparse_attn_step(B, T, ctx, H_I):
    """dsa_sparse_attn_step gives the bits of dsa_index_scores followed by dsa_sparse_attn_select
    (scores, index rows, output), and those match the oracle; three calls in a row."""
    dsa = _dsa()
    _log(f"whole step case B={B} T={T} ctx={ctx} H_I={H_I}")
    H, D, nw, K, ratio, S, DI = 64, 512, 128, 512, 4, 1, 128
    sp = ctx - 1
    g = torch.Generator().manual_seed(B * 13 + T)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    kv_win = torch.randn(B, nw, D, generator=g).to(torch.bfloat16)
    kv_comp = torch.randn(B, T, D, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    qI = torch.randn(B, S, H_I, DI, generator=g).to(torch.bfloat16)
    kI = torch.randn(B, T + 8, DI, generator=g).to(torch.bfloat16)[:, :T]  # batch stride larger than T*DI
    w = (torch.randn(B, S, H_I, generator=g) * 0.5).to(torch.bfloat16)
    scale, w_scale = D ** -0.5, DI ** -0.5 * H_I ** -0.5
    dev = [t.to(DEV) for t in (qI, kI, w, q, kv_win, kv_comp, sink)]
    kw = dict(index_topk=K, start_pos=sp, ratio=ratio, W=nw, scale=scale)
    # the two calls the step stands for
    ref_scores = dsa.dsa_index_scores(dev[0], dev[1], dev[2], w_scale, sp, ratio)
    ref_o, ref_idx = dsa.dsa_sparse_attn_select(ref_scores, *dev[3:], **kw)
    ref_scores, ref_o, ref_idx = ref_scores.cpu().numpy(), ref_o.float().cpu().numpy(), ref_idx.cpu().numpy()
    # against the oracle: scores within the fp32 bound, top-k by the parity rules, attention
    _check_scores(ref_scores, qI, kI.contiguous(), w, w_scale, sp, ratio, ctx="step")
    exp_scores = oracle.index_scores(qI.float().numpy().astype(np.float64), kI.float().numpy().astype(np.float64),
                                     w.float().numpy().astype(np.float64), w_scale, sp, ratio)
    c = int(min(T, oracle.visible_count(0, sp, ratio)))
    win = oracle.window_rows(nw, B, S, sp)
    for b in range(B):
        np.testing.assert_array_equal(ref_idx[b, 0, :win.shape[-1]], win[b, 0])
        check_topk_row(ref_idx[b, 0, win.shape[-1]:], exp_scores[b, 0], min(K, T), c, nw, ctx=f"step ({b},0)")
    exp_o = oracle.sparse_attn(q, oracle.kv_concat(kv_win, kv_comp), sink, ref_idx, scale)
    err = max_abs_err(ref_o, exp_o)
    assert err <= ATTN_TOL["bf16"], err
    for call in range(3):
        o, idx, scores = dsa.dsa_sparse_attn_step(*dev, w_scale=w_scale, **kw)
        n, names = _launched()
        _log(f"  launches: {n} {names}")
        if T <= 2048:
            _assert_one_launch("score+select")
        else:
            assert n >= 3 and "index_scores" in names, names
        np.testing.assert_array_equal(scores.cpu().numpy(), ref_scores)
        np.testing.assert_array_equal(idx.cpu().numpy(), ref_idx)
        np.testing.assert_array_equal(o.float().cpu().numpy(), ref_o)
        _log(f"  call {call}: same bits as the two calls; attention max abs err {err:.3e}")


# ------------------------------------------------------------------------ two-phase decode path
@pytest.mark.parametrize("B,S,L,nc,inval,kernel", [
    (32, 1, 640, 2048, 0.0, "sparse_attn_decode<NS=8>"),
    (24, 1, 640, 1000, 0.1, "sparse_attn_decode<NS=8>"),
    (5, 1, 640, 700, 0.2, "sparse_attn_decode<NS=16>"),    # grid padded to 8 queries
    (16, 1, 640, 16384, 0.0, "sparse_attn_decode<NS=16>"),
    (3, 1, 1000, 900, 0.3, "sparse_attn_bf16"),            # 63 rows per split exceed the decode kernel
    (3, 1, 768, 900, 0.3, "sparse_attn_decode<NS=16>"),    # the longest row the decode kernel takes
    (2, 1, 17, 30, 0.0, "sparse_attn_decode<NS=16>"),      # most splits empty
    (4, 2, 200, 100, 0.5, "sparse_attn_decode<NS=16>"),    # two queries per sequence
])
def test_sparse_attn_decode_path(B, S, L, nc, inval, kernel):
    """H = 64, D = 512 bf16 with few queries: the two-phase kernel where the row fits it (the
    general split kernel otherwise); three calls in a row check that its per-query counters are
    left ready for the next call."""
    dsa = _dsa()
    _log(f"decode path B={B} S={S} L={L} nc={nc} invalid={inval}")
    H, D, nw = 64, 512, 128
    g = torch.Generator().manual_seed(B * 31 + L)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    kv_win = torch.randn(B, nw, D, generator=g).to(torch.bfloat16)
    kv_comp = torch.randn(B, nc, D, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    rng = np.random.default_rng(B + L)
    idx = _rand_idx(rng, B, S, L, nw + nc, frac_invalid=inval)
    idx[0, 0, :] = -1
    scale = D ** -0.5
    kv = oracle.kv_concat(kv_win, kv_comp)
    exp = oracle.sparse_attn(q, kv, sink, idx, scale)
    args = (q.to(DEV), kv_win.to(DEV), kv_comp.to(DEV), sink.to(DEV), torch.from_numpy(idx).to(DEV), scale)
    for call in range(3):
        o = dsa.dsa_sparse_attn(*args)
        n, names = _launched()
        assert names.split("+")[0] == kernel, names
        got = o.float().cpu().numpy()
        err = max_abs_err(got, exp)
        _log(f"  call {call}: max abs err {err:.3e}")
        assert np.all(np.isfinite(got))
        assert np.all(got[0, 0] == 0)
        assert err <= ATTN_TOL["bf16"], err
    assert dsa.dsa_device_errors() == 0


# ------------------------------------------------------------------------ KV sources sliced from larger caches
@pytest.mark.parametrize("B,S,sp,nw,nc,L,fp4,kind", [
    (4, 1, 4095, 128, 1024, 640, False, "sparse_attn_decode<NS="),  # decode kernel
    (2, 200, 0, 200, 75, 200, False, "sparse_attn_prefill"),   # one workgroup per query
    (2, 160, 0, 160, 65, 100, True, "sparse_attn_prefill"),     # fp4 rows and scales sliced
    (2, 2, 0, 40, 30, 77, False, "sparse_attn_bf16"),              # general kernel (H=16)
])
def test_sparse_attn_cache_slices(B, S, sp, nw, nc, L, fp4, kind):
    """KV sources passed as [:B, :n] slices of larger [max_B, max_n, ...] caches (batch stride
    larger than n rows) give the oracle's output over the sliced rows."""
    dsa = _dsa()
    H = 16 if kind == "sparse_attn_bf16" else 64
    D = 512
    _log(f"cache slices B={B} S={S} nw={nw} nc={nc} L={L} fp4={fp4} ({kind})")
    g = torch.Generator().manual_seed(nw + nc + L)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    win_cache = torch.randn(B + 2, nw + 37, D, generator=g).to(torch.bfloat16)
    kv_win = win_cache[:B, :nw]
    sink = torch.randn(H, generator=g)
    if fp4:
        packed, scales = dsa_synth.encode_fp4_e2m1_e4m3(torch.randn(B + 1, nc + 19, D, generator=g), 16)
        comp_rows, comp_sc = packed[:B, :nc], scales[:B, :nc]
        comp64 = oracle.fp4_rows_decode(comp_rows.contiguous(), comp_sc.contiguous())
        comp_dev_full, sc_dev_full = packed.to(DEV), scales.to(DEV)
        comp_dev, sc_dev = comp_dev_full[:B, :nc], sc_dev_full[:B, :nc]
    else:
        comp_cache = torch.randn(B + 3, nc + 50, D, generator=g).to(torch.bfloat16)
        comp_rows = comp_cache[:B, :nc]
        comp64 = comp_rows.contiguous()
        comp_dev_full = comp_cache.to(DEV)
        comp_dev, sc_dev = comp_dev_full[:B, :nc], None
    win_dev_full = win_cache.to(DEV)
    win_dev = win_dev_full[:B, :nw]
    assert win_dev.stride(0) > nw * D and comp_dev.stride(0) > nc * comp_dev.shape[-1]
    rng = np.random.default_rng(L + nc)
    idx = _rand_idx(rng, B, S, L, nw + nc)
    idx[..., -1] = nw + nc - 1  # the last row of the slice
    idx[..., 0] = nw - 1        # the last window row
    o = dsa.dsa_sparse_attn(q.to(DEV), win_dev, comp_dev, sink.to(DEV), torch.from_numpy(idx).to(DEV), D ** -0.5,
                            comp_scales=sc_dev)
    n, names = _launched()
    _log(f"  launches: {n} {names}")
    assert kind in names, names
    exp = oracle.sparse_attn(q, oracle.kv_concat(kv_win.contiguous(), comp64), sink, idx, D ** -0.5)
    err = max_abs_err(o.float().cpu().numpy(), exp)
    _log(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL["bf16"], err


# ------------------------------------------------------------------------ DSA_DEBUG and non-finite inputs
def test_debug_index_check_passes_valid_rows():
    """With the debug index check on, valid index rows (including -1 and the last row) pass and
    give the same output as without it.  (Rows out of range are refused on the host; that path is
    tested on the CPU.)"""
    dsa = _dsa()
    B, S, H, D, nw, nc, L = 2, 3, 64, 512, 40, 60, 90
    g = torch.Generator().manual_seed(5)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16).to(DEV)
    kv_win = torch.randn(B, nw, D, generator=g).to(torch.bfloat16).to(DEV)
    kv_comp = torch.randn(B, nc, D, generator=g).to(torch.bfloat16).to(DEV)
    sink = torch.randn(H, generator=g).to(DEV)
    idx = _rand_idx(np.random.default_rng(3), B, S, L, nw + nc)
    idx[0, 0, 0] = nw + nc - 1
    idx_d = torch.from_numpy(idx).to(DEV)
    ref = dsa.dsa_sparse_attn(q, kv_win, kv_comp, sink, idx_d, D ** -0.5)
    prev = dsa.dsa_set_debug(True)
    try:
        got = dsa.dsa_sparse_attn(q, kv_win, kv_comp, sink, idx_d, D ** -0.5)
    finally:
        dsa.dsa_set_debug(prev)
    assert torch.equal(ref, got)


@pytest.mark.parametrize("B,S,nw,nc,L", [(4, 1, 128, 500, 640), (1, 300, 300, 75, 200), (2, 2, 40, 30, 77)])
def test_nan_in_q_propagates(B, S, nw, nc, L):
    """A NaN in one head's query gives NaN in that head's output, as in the oracle, and leaves every
    other (query, head) finite and correct; the call returns."""
    dsa = _dsa()
    H, D = 64, 512
    g = torch.Generator().manual_seed(B + S + L)
    q = torch.randn(B, S, H, D, generator=g).to(torch.bfloat16)
    q[0, S - 1, 5, 17] = float("nan")
    kv_win = torch.randn(B, nw, D, generator=g).to(torch.bfloat16)
    kv_comp = torch.randn(B, nc, D, generator=g).to(torch.bfloat16)
    sink = torch.randn(H, generator=g)
    idx = _rand_idx(np.random.default_rng(L), B, S, L, nw + nc, frac_invalid=0.0)
    o = dsa.dsa_sparse_attn(q.to(DEV), kv_win.to(DEV), kv_comp.to(DEV), sink.to(DEV), torch.from_numpy(idx).to(DEV),
                            D ** -0.5).float().cpu().numpy()
    with np.errstate(invalid="ignore"):
        exp = oracle.sparse_attn(q, oracle.kv_concat(kv_win, kv_comp), sink, idx, D ** -0.5)
    assert np.all(np.isnan(exp[0, S - 1, 5]))
    assert np.all(np.isnan(o[0, S - 1, 5]))
    mask = np.ones(o.shape[:3], dtype=bool)
    mask[0, S - 1, 5] = False
    assert np.all(np.isfinite(o[mask]))
    assert max_abs_err(o[mask], exp[mask]) <= ATTN_TOL["bf16"]


# ------------------------------------------------------------------------ the page config's ratios (2 and 1)
def _device_set_to_cpu(w, dev_in):
    need = {"q", "kv_win", "kv_comp", "kv_comp_fp4", "kv_comp_scale", "kI", "sink", "qI", "w", "qI_fp4", "qI_scale",
            "kI_fp4", "kI_scale"}
    return {k: v.cpu() for k, v in dev_in.items() if k in need}


@pytest.mark.parametrize("name", ["decode_b16_ctx64k_r2", "decode_b16_ctx64k_r1"])
def test_step_full_real_ratio_decode(name):
    """Decode at 64K context with the ratios of the page's layers (T = 32768 and 65536 index rows
    per query), every query checked: scores, index rows by the parity rules, attention."""
    w = dsa_synth.get(name)
    _log(f"step {name} (full check, T={w.T})")
    dev_in = dsa_synth.generate(w, seed=0, device=DEV)
    o, idx, scores = _step(w, dev_in)
    n, names = _launched()
    _log(f"  launches: {n} {names}")
    # the long rows of a decode batch: the split select (chunk candidates, then their merge)
    assert "topk_split_chunk+topk_split_merge" in names and "sparse_attn_decode<NS=16>" in names, names
    torch.cuda.synchronize()
    cpu_in = _device_set_to_cpu(w, dev_in)
    rows = [(b, t) for b in range(w.B) for t in range(w.S)]
    _check_step(w, cpu_in, o, idx, scores, rows)
    assert _dsa().dsa_device_errors() == 0


@pytest.mark.parametrize("name", ["prefill_s8k_r2", "prefill_s8k_r1"])
def test_step_real_ratio_prefill_sampled(name):
    """Prefill of 8192 tokens with ratios 2 and 1 (T = 4096 and 8192), in the launch configuration
    the benchmark times, on sampled queries (including the c(t) = K crossover)."""
    w = dsa_synth.get(name)
    _log(f"step {name} (full size, sampled, T={w.T})")
    dev_in = dsa_synth.generate(w, seed=0, device=DEV)
    o, idx, scores = _step(w, dev_in)
    n, names = _launched()
    _log(f"  launches: {n} {names}")
    torch.cuda.synchronize()
    cpu_in = _device_set_to_cpu(w, dev_in)
    rows = sample_rows(w, n_random=12)
    _check_step(w, cpu_in, o, idx, scores, rows)


# ------------------------------------------------------------------------ MXFP4 indexer (fp4 q/k, E8M0 per 32)
@pytest.mark.parametrize("B,S,sp,T,H,DI,ratio", [
    (3, 1, 1234, 308, 32, 128, 4),    # decode, ragged 256-row block
    (2, 1, 8191, 2048, 64, 128, 4),   # decode, two MFMA tiles of heads
    (2, 70, 0, 35, 32, 128, 2),       # prefill, several 16-query blocks
    (1, 300, 0, 300, 4, 64, 1),       # few heads (padded to a tile), index head dim 64
    (2, 33, 0, 16, 48, 256, 2),       # index head dim 256
    (1, 130, 5, 1, 32, 128, 4),       # a single compressed row
    (1, 520, 0, 260, 40, 128, 2),
])
def test_index_scores_mxfp4(B, S, sp, T, H, DI, ratio):
    """Scores from packed fp4 index rows with E8M0 block scales against the oracle's decode and
    score definition, within the fp32 accumulation bound; keys passed as a slice of a larger cache."""
    dsa = _dsa()
    _log(f"index_scores_mxfp4 case B={B} S={S} sp={sp} T={T} H={H} DI={DI} r={ratio}")
    g = torch.Generator().manual_seed(S * 11 + T + DI)
    # per-row magnitudes spread over several binades, so the blocks take different scales
    qx = torch.randn(B, S, H, DI, generator=g) * torch.exp2(torch.randint(-3, 4, (B, S, H, 1), generator=g).float())
    kx = torch.randn(B, T + 5, DI, generator=g) * torch.exp2(torch.randint(-3, 4, (B, T + 5, 1), generator=g).float())
    qp, qs = dsa_synth.encode_mxfp4_e8m0(qx, 32)
    kp, ks = dsa_synth.encode_mxfp4_e8m0(kx, 32)
    w = (torch.randn(B, S, H, generator=g) * 0.5).to(torch.bfloat16)
    w_scale = DI ** -0.5 * H ** -0.5
    kp_d, ks_d = kp.to(DEV), ks.to(DEV)
    got = dsa.dsa_index_scores_mxfp4(qp.to(DEV), qs.to(DEV), kp_d[:, :T], ks_d[:, :T], w.to(DEV), w_scale, sp,
                                     ratio).cpu().numpy()
    n, names = _launched()
    assert names == "index_scores_mxfp4", names
    q64 = oracle.mxfp4_rows_decode(qp, qs)
    k64 = oracle.mxfp4_rows_decode(kp[:, :T], ks[:, :T])
    w64 = w.float().numpy().astype(np.float64)
    exp = oracle.index_scores(q64, k64, w64, w_scale, sp, ratio)
    worst = 0.0
    for b in range(B):
        for t in range(S):
            e = exp[b, t]
            inv = np.isinf(e)
            assert np.all(np.isneginf(got[b, t][inv]))
            bound = score_bound(q64[b, t][None], k64[b], w64[b, t][None], w_scale)[0]
            err = np.abs(got[b, t][~inv] - e[~inv])
            lim = 1e-5 * bound[~inv] + 1e-30
            assert np.all(err <= lim), f"({b},{t}): score error {err.max():.3e} above the fp32 bound"
            if err.size:
                worst = max(worst, float((err / lim).max()))
    _log(f"  worst error / bound {worst:.3f}")


@pytest.mark.parametrize("name,full", [("decode_b32_ctx8k_mxfp4", True), ("decode_b16_ctx64k_mxfp4", True),
                                       ("decode_b16_ctx64k_r1_mxfp4", True), ("prefill_s8k_mxfp4", False)])
def test_step_mxfp4(name, full):
    """The whole step with the MXFP4 indexer at full size: every decode query, sampled prefill
    queries (scores, index rows by the parity rules, attention)."""
    w = dsa_synth.get(name)
    _log(f"step {name} ({'full check' if full else 'sampled'}, T={w.T})")
    dev_in = dsa_synth.generate(w, seed=0, device=DEV)
    o, idx, scores = _step(w, dev_in)
    n, names = _launched()
    _log(f"  launches: {n} {names}")
    assert names.startswith("index_scores_mxfp4+"), names
    torch.cuda.synchronize()
    cpu_in = _device_set_to_cpu(w, dev_in)
    rows = [(b, t) for b in range(w.B) for t in range(w.S)] if full else sample_rows(w, n_random=12)
    _check_step(w, cpu_in, o, idx, scores, rows)
    assert _dsa().dsa_device_errors() == 0


# ------------------------------------------------------------------------ two-level selection (candidate blocks)
def _unpack_bits(words, nblk):
    w = np.asarray(words).astype(np.int64) & 0xFFFFFFFF
    bits = (w[..., :, None] >> np.arange(32)) & 1
    flat = bits.reshape(*w.shape[:-1], -1).astype(bool)
    return flat[..., :nblk], flat[..., nblk:]


def _pack_bits(blocks):
    """bool [..., nblk] -> int32 words [..., ceil(nblk/32)] (bit i%32 of word i/32)."""
    nblk = blocks.shape[-1]
    nw = (nblk + 31) // 32
    pad = np.zeros(blocks.shape[:-1] + (nw * 32,), dtype=np.uint64)
    pad[..., :nblk] = blocks
    words = (pad.reshape(*blocks.shape[:-1], nw, 32) << np.arange(32, dtype=np.uint64)).sum(-1)
    return words.astype(np.uint32).view(np.int32)


@pytest.mark.parametrize("B,S,T,sp,ratio,bs,nsel,kind", [
    (4, 1, 65536, 65535, 1, 8, 2048, "normal"),  # the page's candidate source: ratio 1 at 64K context
    (2, 1, 32768, 65535, 2, 8, 2048, "ties"),
    (1, 300, 1000, 0, 1, 8, 20, "normal"),       # prefill rows: blocks partly visible
    (3, 2, 777, 3099, 4, 4, 50, "ties"),
    (2, 1, 100, 399, 4, 8, 100, "normal"),       # every visible block fits
])
def test_candidate_blocks(B, S, T, sp, ratio, bs, nsel, kind):
    """Given the same float32 scores, the chosen blocks equal the oracle's bit for bit (padding bits
    of a row's last word stay zero)."""
    dsa = _dsa()
    _log(f"candidate blocks B={B} S={S} T={T} sp={sp} r={ratio} bs={bs} nsel={nsel} {kind}")
    rng = np.random.default_rng(T + nsel)
    s = (rng.integers(-4, 5, size=(B, S, T)).astype(np.float32) if kind == "ties"
         else rng.standard_normal((B, S, T)).astype(np.float32))
    c = np.minimum(oracle.visible_count(np.arange(S), sp, ratio), T)
    s[:, np.arange(T)[None, :] >= c[:, None]] = -np.inf
    bits = dsa.dsa_candidate_blocks(torch.from_numpy(s).to(DEV), sp, ratio, bs, nsel)
    assert _launched()[1] == "candidate_blocks"
    nblk = -(-T // bs)
    got, padbits = _unpack_bits(bits.cpu().numpy(), nblk)
    assert not padbits.any()
    for b in range(B):
        for t in range(S):
            exp = oracle.candidate_blocks_row(s[b, t].astype(np.float64), int(c[t]), nsel, bs)
            np.testing.assert_array_equal(got[b, t], exp, err_msg=f"row ({b},{t})")


@pytest.mark.parametrize("B,S,sp,T,H,DI,ratio,bs,nsel,fmt", [
    (4, 1, 65535, 16384, 32, 128, 4, 8, 300, "bf16"),  # decode: keys outside the candidates are not read
    (2, 70, 0, 70, 32, 128, 1, 8, 5, "bf16"),          # 16 queries per block
    (1, 200, 37, 130, 20, 128, 1, 4, 10, "bf16"),      # the key-streaming prefill kernel
    (1, 9, 0, 9, 4, 32, 1, 2, 2, "f32"),
    (3, 1, 4000, 1000, 32, 128, 4, 8, 30, "mxfp4"),
    (1, 100, 0, 100, 32, 128, 1, 8, 4, "mxfp4"),
])
def test_index_scores_masked(B, S, sp, T, H, DI, ratio, bs, nsel, fmt):
    """A consumer layer's scores inside the candidate blocks (the oracle's scores there, -inf
    elsewhere), with candidates the oracle chose from another layer's scores."""
    dsa = _dsa()
    _log(f"masked index scores B={B} S={S} sp={sp} T={T} H={H} DI={DI} r={ratio} bs={bs} nsel={nsel} {fmt}")
    g = torch.Generator().manual_seed(T * 3 + S + nsel)
    src = torch.randn(B, S, T, generator=g).double().numpy()
    mask = oracle.candidate_mask(src, sp, ratio, nsel, bs)
    nblk = -(-T // bs)
    blocks = np.zeros((B, S, nblk), dtype=bool)
    c = oracle.visible_count(np.arange(S), sp, ratio)
    for b in range(B):
        for t in range(S):
            blocks[b, t] = oracle.candidate_blocks_row(src[b, t], int(min(T, c[t])), nsel, bs)
    cand = (torch.from_numpy(_pack_bits(blocks)).to(DEV), bs)
    w = (torch.randn(B, S, H, generator=g) * 0.5)
    w_scale = DI ** -0.5 * H ** -0.5
    if fmt == "mxfp4":
        qp, qs = dsa_synth.encode_mxfp4_e8m0(torch.randn(B, S, H, DI, generator=g), 32)
        kp, ks = dsa_synth.encode_mxfp4_e8m0(torch.randn(B, T, DI, generator=g), 32)
        wb = w.to(torch.bfloat16)
        got = dsa.dsa_index_scores_mxfp4(qp.to(DEV), qs.to(DEV), kp.to(DEV), ks.to(DEV), wb.to(DEV), w_scale, sp,
                                         ratio, candidates=cand).cpu().numpy()
        q64, k64 = oracle.mxfp4_rows_decode(qp, qs), oracle.mxfp4_rows_decode(kp, ks)
        w64 = wb.float().numpy().astype(np.float64)
    else:
        dt = torch.float32 if fmt == "f32" else torch.bfloat16
        qI = torch.randn(B, S, H, DI, generator=g).to(dt)
        kI = torch.randn(B, T, DI, generator=g).to(dt)
        wd = w.to(dt)
        got = dsa.dsa_index_scores_masked(qI.to(DEV), kI.to(DEV), wd.to(DEV), w_scale, sp, ratio, cand).cpu().numpy()
        q64, k64 = qI.float().numpy().astype(np.float64), kI.float().numpy().astype(np.float64)
        w64 = wd.float().numpy().astype(np.float64)
    _log(f"  launches: {_launched()}")
    exp = np.where(mask, oracle.index_scores(q64, k64, w64, w_scale, sp, ratio), -np.inf)
    for b in range(B):
        for t in range(S):
            e = exp[b, t]
            inv = np.isinf(e)
            assert np.all(np.isneginf(got[b, t][inv])), f"({b},{t}): outside the candidates must be -inf"
            bound = score_bound(q64[b, t][None], k64[b], w64[b, t][None], w_scale)[0]
            assert np.all(np.abs(got[b, t][~inv] - e[~inv]) <= 1e-5 * bound[~inv] + 1e-30), (b, t)


def _check_blocks_banded(chosen, scores_row, c, nsel, bs, ctx):
    """The chosen blocks are a valid pick for oracle scores that differ from the GPU's by rounding:
    exactly min(nsel, visible blocks) of them, and blocks on either side of the threshold only
    within 1e-3 relative of it."""
    cb = -(-c // bs)
    bmax = np.array([scores_row[i * bs:min((i + 1) * bs, c)].max() for i in range(cb)])
    n = min(nsel, cb)
    assert chosen[:cb].sum() == n and not chosen[cb:].any(), ctx
    if cb <= nsel:
        return
    order = np.sort(bmax)[::-1]
    sk, sk1 = order[n - 1], order[n]
    delta = 1e-3 * max(abs(sk), abs(sk1))
    assert np.all(bmax[chosen[:cb]] >= sk - delta), ctx
    assert np.all(bmax[~chosen[:cb]] <= sk + delta), ctx


@pytest.mark.parametrize("name", ["decode_b16_ctx64k_r1", "decode_b16_ctx64k_r1_mxfp4"])
def test_two_level_step(name):
    """The page's two-level selection at its real shape (ratio 1, 64K context, 2048 blocks of 8):
    the source layer's scores give the candidate blocks; a consumer layer scores inside them with
    its own index queries and weights, selects and attends.  Candidates are checked against the
    oracle's source scores by the banded rule, the consumer's index rows and attention against the
    oracle given those candidates."""
    dsa = _dsa()
    w = dsa_synth.get(name)
    bs, nsel = 8, 2048
    _log(f"two-level step {name}: T={w.T}, {nsel} blocks of {bs}")
    src = dsa_synth.generate(w, seed=0, device=DEV)   # the candidate source layer
    con = dsa_synth.generate(w, seed=1, device=DEV)   # a consumer layer (own q, index q, weights)
    w_scale = w.D_I ** -0.5 * w.H_I ** -0.5
    mx = w.index_fmt == "mxfp4"
    if mx:
        s_src = dsa.dsa_index_scores_mxfp4(src["qI_fp4"], src["qI_scale"], src["kI_fp4"], src["kI_scale"], src["w"],
                                           w_scale, w.start_pos, w.ratio)
    else:
        s_src = dsa.dsa_index_scores(src["qI"], src["kI"], src["w"], w_scale, w.start_pos, w.ratio)
    bits = dsa.dsa_candidate_blocks(s_src, w.start_pos, w.ratio, bs, nsel)
    # the consumer reads the source's index keys and compressed KV (shared caches) with its own queries
    if mx:
        s_con = dsa.dsa_index_scores_mxfp4(con["qI_fp4"], con["qI_scale"], src["kI_fp4"], src["kI_scale"], con["w"],
                                           w_scale, w.start_pos, w.ratio, candidates=(bits, bs))
    else:
        s_con = dsa.dsa_index_scores_masked(con["qI"], src["kI"], con["w"], w_scale, w.start_pos, w.ratio, (bits, bs))
    o, idx = dsa.dsa_sparse_attn_select(s_con, con["q"], con["kv_win"], src["kv_comp"], con["sink"],
                                        index_topk=w.index_topk, start_pos=w.start_pos, ratio=w.ratio, W=w.W,
                                        scale=w.D ** -0.5)
    torch.cuda.synchronize()
    cpu_src = _device_set_to_cpu(w, src)
    cpu_con = _device_set_to_cpu(w, con)
    q64s, k64 = _index_f64(cpu_src)
    q64c, _ = _index_f64(cpu_con)
    c = int(min(w.T, oracle.visible_count(0, w.start_pos, w.ratio)))
    nblk = -(-w.T // bs)
    got_blocks, _ = _unpack_bits(bits.cpu().numpy(), nblk)
    exp_src = oracle.index_scores(q64s, k64, cpu_src["w"].float().numpy().astype(np.float64), w_scale, w.start_pos,
                                  w.ratio)
    exp_con = oracle.index_scores(q64c, k64, cpu_con["w"].float().numpy().astype(np.float64), w_scale, w.start_pos,
                                  w.ratio)
    idx_cpu = idx.cpu().numpy()
    win = oracle.window_rows(w.W, w.B, w.S, w.start_pos)
    rules = {}
    for b in range(w.B):
        _check_blocks_banded(got_blocks[b, 0], exp_src[b, 0], c, nsel, bs, f"({b},0) blocks")
        mask = np.repeat(got_blocks[b, 0], bs)[:w.T] & (np.arange(w.T) < c)
        masked = np.where(mask, exp_con[b, 0], -np.inf)
        np.testing.assert_array_equal(idx_cpu[b, 0, :w.Wc], win[b, 0])
        sel = idx_cpu[b, 0, w.Wc:]
        assert np.all(mask[sel[sel >= 0] - w.n_win]), "a selected row outside the candidate blocks"
        rule = check_topk_row(sel, masked, w.K, c, w.n_win, ctx=f"{name} ({b},0)")
        rules[rule] = rules.get(rule, 0) + 1
    kv = oracle.kv_concat(cpu_con["kv_win"], cpu_src["kv_comp"])
    exp_o = oracle.sparse_attn(cpu_con["q"], kv, cpu_con["sink"], idx_cpu, w.D ** -0.5)
    err = max_abs_err(o.float().cpu().numpy(), exp_o)
    _log(f"  top-k rules {rules}, attention max abs err {err:.3e}")
    assert err <= ATTN_TOL["bf16"], err


# ------------------------------------------------------------------------ output epilogue and cache write
@pytest.mark.parametrize("B,S,H,D,nw,nc,L,rd,dtype,fp4,kernel", [
    (4, 1, 64, 512, 128, 600, 640, 64, "bf16", False, "sparse_attn_decode<NS=16>"),  # fused epilogue
    (32, 1, 64, 512, 128, 2048, 640, 64, "bf16", False, "sparse_attn_decode<NS=8>"),
    (1, 300, 64, 512, 300, 75, 200, 64, "bf16", False, "sparse_attn_prefill"),    # fused epilogue
    (1, 260, 64, 512, 260, 65, 100, 128, "bf16", True, "sparse_attn_prefill"),
    (2, 3, 16, 512, 40, 30, 77, 64, "bf16", False, "sparse_attn_bf16"),               # separate pass
    (1, 5, 4, 64, 20, 16, 24, 16, "f32", False, "sparse_attn_f32"),
])
def test_sparse_attn_rope(B, S, H, D, nw, nc, L, rd, dtype, fp4, kernel):
    """The attention output with its inverse rotary embedding (`Attention.forward`) against the
    oracle's exact attention followed by its exact inverse rotation."""
    dsa = _dsa()
    _log(f"attention + inverse rope B={B} S={S} H={H} D={D} L={L} rd={rd} {dtype} fp4={fp4}")
    g = torch.Generator().manual_seed(B + S + L + rd)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    q = torch.randn(B, S, H, D, generator=g).to(dt)
    kv_win = torch.randn(B, nw, D, generator=g).to(dt)
    sink = torch.randn(H, generator=g)
    if fp4:
        packed, scales = dsa_synth.encode_fp4_e2m1_e4m3(torch.randn(B, nc, D, generator=g), 16)
        comp64, comp_dev, sc_dev = oracle.fp4_rows_decode(packed, scales), packed.to(DEV), scales.to(DEV)
    else:
        comp = torch.randn(B, nc, D, generator=g).to(dt)
        comp64, comp_dev, sc_dev = comp, comp.to(DEV), None
    idx = _rand_idx(np.random.default_rng(L), B, S, L, nw + nc)
    freqs = dsa_synth.rope_freqs(np.arange(S) + 1000 * (S == 1) * 8 + 17, rd)
    o = dsa.dsa_sparse_attn_rope(q.to(DEV), kv_win.to(DEV), comp_dev, sink.to(DEV), torch.from_numpy(idx).to(DEV),
                                 D ** -0.5, freqs.to(DEV), comp_scales=sc_dev)
    n, names = _launched()
    _log(f"  launches: {n} {names}")
    assert names.startswith(kernel), names
    if kernel in ("sparse_attn_decode<NS=16>", "sparse_attn_decode<NS=8>", "sparse_attn_prefill"):
        assert n == 1, names  # rotated in the attention kernel's epilogue
    else:
        assert names.endswith("rope_inverse"), names
    exp = oracle.rope_rotate(oracle.sparse_attn(q, oracle.kv_concat(kv_win, comp64), sink, idx, D ** -0.5),
                             freqs.numpy(), inverse=True)
    err = max_abs_err(o.float().cpu().numpy(), exp)
    _log(f"  max abs err {err:.3e}")
    assert err <= ATTN_TOL[dtype], err


@pytest.mark.parametrize("B,n,D,rd,row0,R", [(2, 37, 512, 64, 5, 50), (1, 8192, 512, 64, 0, 8192),
                                             (3, 3, 64, 16, 11, 20)])
def test_compress_kv_write(B, n, D, rd, row0, R):
    """`_compress_kv`'s cache write: rotated, quantised and stored bytes equal the oracle's bit for
    bit (every code is decided in the page's float32 steps), rows outside [row0, row0+n) untouched."""
    dsa = _dsa()
    _log(f"compress kv write B={B} n={n} D={D} rd={rd} rows {row0}..{row0 + n} of {R}")
    g = torch.Generator().manual_seed(n + D + row0)
    lat = (torch.randn(B, n, D, generator=g) * torch.exp(torch.randn(B, n, 1, generator=g))).to(torch.bfloat16)
    # a group of exact e2m1 midpoints (scale 2^-1 from amax 3): the ties go to the even code
    if D - rd >= 16:
        lat[0, 0, :16] = torch.tensor([3.0, 0.125, 0.375, 0.625, 0.875, 1.25, 1.75, 2.5,
                                       -0.125, -0.375, -1.25, -2.5, 0.0, -0.0, 1.0, -3.0]).to(torch.bfloat16)
    freqs = dsa_synth.rope_freqs(np.arange(n) * 4 + 3, rd)
    rows = torch.full((B, R, D // 2), 0xAB, dtype=torch.uint8, device=DEV)
    scales = torch.full((B, R, D // 16), 0xCD, dtype=torch.uint8, device=DEV)
    dsa.dsa_compress_kv_write(lat.to(DEV), freqs.to(DEV), rows, scales, row0)
    assert _launched()[1] == "compress_kv_write"
    exp_p, exp_s = oracle.compress_kv_write(lat.float().numpy(), freqs.numpy(), rd)
    got_p, got_s = rows.cpu().numpy(), scales.cpu().numpy()
    np.testing.assert_array_equal(got_p[:, row0:row0 + n], exp_p)
    np.testing.assert_array_equal(got_s[:, row0:row0 + n], exp_s)
    assert np.all(got_p[:, :row0] == 0xAB) and np.all(got_p[:, row0 + n:] == 0xAB)
    assert np.all(got_s[:, :row0] == 0xCD) and np.all(got_s[:, row0 + n:] == 0xCD)
