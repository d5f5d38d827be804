"""Benchmark of the sparse MQA attention step on one MI355X.

A step is one pass of the whole path over one batch of synthetic input through
dsa_sparse_attn_step: index scores, index rows (window rows and top-k selection) and sparse
attention.  For decode batches the library runs that as one kernel; otherwise it is three launches
(index scores, index rows, attention), every one a libdsa kernel.  Which kernels ran is read back
from the library (dsa_last_launches), not assumed.  Inputs are resident in HBM before timing
starts; several input sets are rotated so that the 256 MB Infinity Cache cannot serve one step
from the previous one.

Default run: every bf16 workload (decode_b32_ctx8k, prefill_s8k, decode_b16_ctx64k,
prefill_s32k_fp4, and the page config's ratios 2 and 1 at 64K-context decode and 8K prefill) in one
process, then ONE JSON line whose headline (value, config, roofline, cpu_baseline) is the largest,
prefill_s32k_fp4, and whose "workloads" object carries each workload's step time, kernels and
roofline.  Some workloads are also timed as a layer group: one step on the index source layer
plus the attention of the layers that reuse its index rows.  The roofline covers each workload's dominant kernel
(the one-launch decode step, or the sparse attention kernel): `achieved` is its algorithmic work
per launch over its average duration in a graph of 100 back-to-back launches, timed with HIP events
on the stream it runs on; `median_launch_us` is the median of 100 launches timed one by one.  The
CPU baseline is the oracle, timed on a bounded sample of the headline workload on the host.

Calibration modes (each prints one JSON line and exits):
  --copy-calibration MIB   a plain device copy of MIB MiB, three times (scale of the HBM byte counters)
  --calibrate              attainable figures on this GPU: streaming copy bandwidth, a large bf16
                           GEMM (hipBLASLt through torch) and the per-launch floor of a tiny kernel
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn query-tokens/s (decode & prefill) at 1 GPU; % HBM / MFMA peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
ROTATE_BYTES = 768 << 20  # rotate input sets until they span more than the Infinity Cache (256 MB)
HEADLINE = "prefill_s32k_fp4"  # the largest workload
LINE_WORKLOADS = ["decode_b32_ctx8k", "prefill_s8k", "decode_b16_ctx64k", "prefill_s32k_fp4",
                  "decode_b16_ctx64k_r2", "decode_b16_ctx64k_r1", "prefill_s8k_r2", "prefill_s8k_r1",
                  "decode_b32_ctx8k_mxfp4", "decode_b16_ctx64k_mxfp4", "decode_b16_ctx64k_r1_mxfp4",
                  "prefill_s8k_mxfp4"]
# workloads also timed as a layer group: one index source layer and the layers that reuse its index
# rows (the page's index sources sit every 4 layers from layer 20 on, all reading layer 20's
# compressed KV), each layer with its own queries, window KV and sinks
GROUP_LAYERS = 4
# workloads where the two-level selection is timed: the page's candidate source (layer 20, ratio 1)
# keeps 2048 blocks of 8 compressed positions, and the later index sources score only inside them
TWO_LEVEL = {"decode_b16_ctx64k_r1": (8, 2048), "decode_b16_ctx64k_r1_mxfp4": (8, 2048)}
GROUP_WORKLOADS = ["decode_b32_ctx8k", "decode_b16_ctx64k_r2", "decode_b16_ctx64k_r1", "prefill_s8k_r1",
                   "decode_b16_ctx64k_r1_mxfp4"]
HOST_CORES = 16  # the CPU share of one GPU on the benchmark machines
# the sources each dominant kernel is compiled from: a change to any of them drops the HBM traffic
# figure taken on the old sources
KERNEL_SOURCES = {
    "decode": ["sparse_mqa_attention_amd/csrc/sparse_attn_decode.hip", "sparse_mqa_attention_amd/csrc/dsa_internal.h",
               "sparse_mqa_attention_amd/csrc/topk_block.h", "sparse_mqa_attention_amd/csrc/index_tile.h"],
    "prefill": ["sparse_mqa_attention_amd/csrc/sparse_attn_prefill.hip",
                "sparse_mqa_attention_amd/csrc/dsa_internal.h"],
}


def _args():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100, help="timed steps per workload")
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="all", help="one workload name, or 'all' (the default line)")
    p.add_argument("--launches", type=int, default=100, help="dominant-kernel launches timed for avg and median")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB three times (scale of the HBM byte counters)")
    p.add_argument("--calibrate", action="store_true", help="only measure attainable copy, GEMM and launch figures")
    return p.parse_args()


# ---------------------------------------------------------------------------- calibration modes
def copy_calibration(mib: int):
    """A plain device-to-device copy of known size, three times: reads and writes mib MiB each."""
    import torch

    n = mib << 20
    x = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)


def _graph_time_ms(fn, reps: int, inner: int):
    """Average ms of fn() over `inner` calls captured in one graph, replayed `reps` times."""
    import torch

    stream = torch.cuda.current_stream()
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(inner):
            fn()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * inner)


def calibrate():
    """Attainable figures on this GPU, each timed with HIP events over graphs of back-to-back calls."""
    import torch

    dev = torch.device("cuda:0")
    out = {"calibration": "MI355X attainable figures"}
    # streaming copy: 2 GiB read + 2 GiB written per call
    n = 2 << 30
    x = torch.ones(n, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    ms = _graph_time_ms(lambda: y.copy_(x), reps=5, inner=4)
    out["copy_bytes_per_call"] = 2 * n
    out["copy_gbs"] = round(2 * n / (ms * 1e-3) / 1e9, 1)
    del x, y
    # dense bf16 GEMM 8192 x 8192 x 8192 through torch (hipBLASLt)
    m = 8192
    a = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    b = torch.randn(m, m, device=dev, dtype=torch.bfloat16)
    c = torch.empty(m, m, device=dev, dtype=torch.bfloat16)
    ms = _graph_time_ms(lambda: torch.matmul(a, b, out=c), reps=5, inner=4)
    out["gemm_shape"] = [m, m, m]
    out["gemm_bf16_tflops"] = round(2.0 * m ** 3 / (ms * 1e-3) / 1e12, 1)
    del a, b, c
    # launch floor: a one-workgroup fill kernel, 100 back to back in a graph
    z = torch.empty(64, device=dev)
    out["tiny_kernel_us_back_to_back"] = round(_graph_time_ms(lambda: z.fill_(1.0), reps=5, inner=100) * 1e3, 3)
    # a 256-workgroup fill (256 x 1 KiB)
    z2 = torch.empty(256 * 256, device=dev)
    out["fill_256_workgroups_us_back_to_back"] = round(
        _graph_time_ms(lambda: z2.fill_(1.0), reps=5, inner=100) * 1e3, 3)
    out["peaks_used"] = {"hbm_gbs": PEAK_HBM_GBS, "bf16_tflops": PEAK_BF16_TFLOPS}
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------------------- traffic records
def kernel_src_sha(mode: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[mode]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _traffic(workload: str, sha: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if taken on this kernel source."""
    path = os.path.join(ROOT, "profiles", f"sparse_attn_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_src_sha") != sha:
        return None
    return d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------- CPU baseline
_ORACLE_JOB = {}  # filled before the worker pool forks; workers read it, only (b, t) is sent


def _oracle_query(bt):
    """The oracle's whole path for one query: scores, top-k, window+top-k row, attention."""
    import numpy as np

    import oracle

    g = _ORACLE_JOB
    w = g["w"]
    b, t = bt
    sp = w.start_pos + t  # absolute position of the query; row (0, 0) of the one-query views below
    s = oracle.index_scores_rows(g["qI"][b, t][None, None], g["kI"][b][None], g["wt"][b, t][None, None],
                                 g["w_scale"], sp, w.ratio, [(0, 0)])[0]
    c = int(min(w.T, oracle.visible_count(0, sp, w.ratio)))
    sel = oracle.topk_select_row(s, w.K, c, w.n_win)
    idx = np.concatenate([g["win"][t], sel])
    return oracle.sparse_attn_rows(g["q"][b, t][None, None], g["kv"][b][None], g["sink"], idx[None, None],
                                   w.D ** -0.5, [(0, 0)])[0]


def _pool_init():
    for v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[v] = "1"


def cpu_baseline(w, cpu_in, target_s: float):
    """Time the oracle (scores, top-k, window rows, attention) on a sample of the workload's
    queries over a process pool; returns the baseline object."""
    import multiprocessing as mp

    import numpy as np

    import oracle

    # every host core the machine gives one GPU: the benchmark machines grant 16 per GPU whatever
    # os.cpu_count() reports, so the pool never exceeds that
    cores = max(1, min(HOST_CORES, os.cpu_count() or 1))
    comp = (oracle.fp4_rows_decode(cpu_in["kv_comp_fp4"], cpu_in["kv_comp_scale"]) if w.comp_fmt == "fp4"
            else cpu_in["kv_comp"])
    f64 = lambda x: x.float().numpy().astype(np.float64)  # noqa: E731
    if "qI_fp4" in cpu_in:  # the MXFP4 indexer: the oracle decodes the packed rows
        qI = oracle.mxfp4_rows_decode(cpu_in["qI_fp4"], cpu_in["qI_scale"])
        kI = oracle.mxfp4_rows_decode(cpu_in["kI_fp4"], cpu_in["kI_scale"])
    else:
        qI, kI = f64(cpu_in["qI"]), f64(cpu_in["kI"])
    _ORACLE_JOB.update(w=w, kv=oracle.kv_concat(cpu_in["kv_win"], comp), win=oracle.window_rows(w.W, 1, w.S,
                       w.start_pos)[0], sink=f64(cpu_in["sink"]), qI=qI, kI=kI,
                       wt=f64(cpu_in["w"]), q=cpu_in["q"], w_scale=w.D_I ** -0.5 * w.H_I ** -0.5)
    rng = np.random.default_rng(0)
    order = [(b, t) for b in range(w.B) for t in range(w.S)]
    rng.shuffle(order)
    done = 0
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores, initializer=_pool_init) as pool:
        i = 0
        while time.perf_counter() - t0 < target_s and done < len(order):
            batch = [order[(i + k) % len(order)] for k in range(2 * cores)]
            i += len(batch)
            pool.map(_oracle_query, batch, chunksize=1)
            done += len(batch)
    el = time.perf_counter() - t0
    _ORACLE_JOB.clear()
    return {"value": round(done / el, 2), "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} distinct queries of {w.name} drawn at random, each the oracle's scores + top-k + "
                      f"window row + attention in float64 NumPy, {cores} worker processes x 1 BLAS thread "
                      f"(the host-core share of one GPU), {el:.1f} s wall"}


# ---------------------------------------------------------------------------- one workload
def visible_pairs(w) -> int:
    """Visible (query, compressed row) pairs of the step: sum over queries of min(T, c(t))."""
    tot = 0
    for t in range(w.S):
        tot += min(w.T, (w.start_pos + t + 1) // w.ratio)
    return w.B * tot


def run_workload(w, a, log):
    """Times one workload's step and dominant kernel; returns (entry dict, set 0 inputs)."""
    import torch

    import dsa_synth
    import sparse_mqa_attention_amd as dsa

    dev = torch.device("cuda:0")
    set0 = dsa_synth.generate(w, seed=0, device=dev)
    set_bytes = sum(dsa_synth.nbytes(t) for t in set0.values())
    n_sets = max(1, min(8, math.ceil(ROTATE_BYTES / set_bytes)))
    sets = [set0] + [dsa_synth.generate(w, seed=s, device=dev) for s in range(1, n_sets)]
    scale = w.D ** -0.5
    w_scale = w.D_I ** -0.5 * w.H_I ** -0.5
    Wc = dsa.dsa_window_cols(w.S, w.start_pos, w.W)
    dcode = 1 if w.dtype == "bf16" else 0
    bufs = []
    for s in sets:
        ws = dsa.dsa_step_workspace_size(dcode, w.B, w.S, w.H, w.D, w.T, w.index_topk, w.start_pos, w.W)
        bufs.append({"idx": torch.empty(w.B, w.S, Wc + w.K, dtype=torch.int32, device=dev),
                     "scores": torch.empty(w.B, w.S, w.T, dtype=torch.float32, device=dev),
                     "o": torch.empty_like(s["q"]),
                     "workspace": torch.zeros(max(ws, 1), dtype=torch.uint8, device=dev)})
    stream = torch.cuda.current_stream(dev)
    comp_key = "kv_comp_fp4" if w.comp_fmt == "fp4" else "kv_comp"

    mx = w.index_fmt == "mxfp4"

    def step(i):
        s, bf = sets[i % n_sets], bufs[i % n_sets]
        kw = dict(index_topk=w.index_topk, start_pos=w.start_pos, ratio=w.ratio, W=w.W, scale=scale, w_scale=w_scale,
                  comp_scales=s.get("kv_comp_scale"), out=bf["o"], scores=bf["scores"], idx=bf["idx"],
                  workspace=bf["workspace"])
        if mx:
            dsa.dsa_sparse_attn_step_mxfp4(s["qI_fp4"], s["qI_scale"], s["kI_fp4"], s["kI_scale"], s["w"], s["q"],
                                           s["kv_win"], s[comp_key], s["sink"], **kw)
        else:
            dsa.dsa_sparse_attn_step(s["qI"], s["kI"], s["w"], s["q"], s["kv_win"], s[comp_key], s["sink"], **kw)

    def index(i):
        s, bf = sets[i % n_sets], bufs[i % n_sets]
        if mx:
            dsa.dsa_index_scores_mxfp4(s["qI_fp4"], s["qI_scale"], s["kI_fp4"], s["kI_scale"], s["w"], w_scale,
                                       w.start_pos, w.ratio, out=bf["scores"])
        else:
            dsa.dsa_index_scores(s["qI"], s["kI"], s["w"], w_scale, w.start_pos, w.ratio, out=bf["scores"])

    def attn(i):
        s, bf = sets[i % n_sets], bufs[i % n_sets]
        dsa.dsa_sparse_attn(s["q"], s["kv_win"], s[comp_key], s["sink"], bf["idx"], scale,
                            comp_scales=s.get("kv_comp_scale"), out=bf["o"], workspace=bf["workspace"])

    def rest(i):
        s, bf = sets[i % n_sets], bufs[i % n_sets]
        index(i)
        dsa.dsa_select(bf["scores"], w.index_topk, w.start_pos, w.ratio, w.W, w.n_win, out=bf["idx"],
                       workspace=bf["workspace"])

    # eager warmup (initialises every set) and the library's own record of what a step launches
    for i in range(max(n_sets, min(a.warmup, 2 * n_sets))):
        step(i)
    n_launch, names = dsa.dsa_last_launches()
    torch.cuda.synchronize()
    fused = n_launch == 1  # the whole step in one kernel (read back from the library)

    def capture(fn, first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(count):
                fn(first + k)
        return g

    # K steps: graphs of G consecutive steps (rotating input sets), bracketed by HIP events
    G = max(1, min(a.steps, 10))
    full = capture(step, 0, G)
    rem = a.steps % G
    tail = capture(step, 0, rem) if rem else None
    for _ in range(max(1, a.warmup // G)):
        full.replay()
    torch.cuda.synchronize()
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(a.steps // G):
        full.replay()
    if tail is not None:
        tail.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms_per_step = t_start.elapsed_time(t_end) / a.steps
    del full, tail

    # the dominant kernel: R launches back to back in one graph (average), and R launches timed one
    # by one (median), each on the launch stream
    dominant = step if fused else attn
    dominant(0)
    dom_names = dsa.dsa_last_launches()[1]
    R = a.launches
    g_avg = capture(dominant, 0, R)
    g_avg.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    g_avg.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    avg_ms = e0.elapsed_time(e1) / R
    del g_avg
    singles = [capture(dominant, i, 1) for i in range(n_sets)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    for i in range(R):
        evs[i].record(stream)
        singles[i % n_sets].replay()
    evs[R].record(stream)
    torch.cuda.synchronize()
    med_ms = statistics.median(evs[i].elapsed_time(evs[i + 1]) for i in range(R))
    del singles
    rest_ms = index_ms = None
    if not fused:
        rest_ms = _graph_time_ms(lambda: rest(0), reps=2, inner=20)
        index_ms = _graph_time_ms(lambda: index(0), reps=2, inner=20)

    # the two-level selection: candidate blocks from this step's scores, then a consumer layer's
    # index scores inside them (the same index queries here; only the keys read differ)
    two_level = None
    if w.name in TWO_LEVEL:
        bs, nsel = TWO_LEVEL[w.name]
        s0, b0 = sets[0], bufs[0]
        nw = ((w.T + bs - 1) // bs + 31) // 32
        bits = torch.empty(w.B, w.S, nw, dtype=torch.int32, device=dev)
        masked = torch.empty_like(b0["scores"])

        def cand_blocks():
            dsa.dsa_candidate_blocks(b0["scores"], w.start_pos, w.ratio, bs, nsel, out=bits)

        def consumer():
            if mx:
                dsa.dsa_index_scores_mxfp4(s0["qI_fp4"], s0["qI_scale"], s0["kI_fp4"], s0["kI_scale"], s0["w"], w_scale,
                                           w.start_pos, w.ratio, out=masked, candidates=(bits, bs))
            else:
                dsa.dsa_index_scores_masked(s0["qI"], s0["kI"], s0["w"], w_scale, w.start_pos, w.ratio, (bits, bs),
                                            out=masked)

        step(0)
        cb_ms = _graph_time_ms(cand_blocks, reps=2, inner=20)
        cons_ms = _graph_time_ms(consumer, reps=2, inner=20)
        kept = float(torch.stack([((bits >> k) & 1).sum() for k in range(32)]).sum().item()) / (w.B * w.S)
        two_level = {"block_size": bs, "blocks_kept": nsel, "candidate_blocks_us": round(cb_ms * 1e3, 2),
                     "masked_index_us": round(cons_ms * 1e3, 2), "full_index_us": round(index_ms * 1e3, 2),
                     "blocks_chosen_per_query": kept}
        del bits, masked

    # a layer group: the step on the index source layer, then the attention of the layers that reuse
    # its index rows (own queries, window KV and sinks; the shared compressed KV)
    group = None
    if w.name in GROUP_WORKLOADS:
        layers = []
        for li in range(1, GROUP_LAYERS):
            g = dsa_synth.generate(w, seed=1000 + li, device=dev)
            layers.append({"q": g["q"], "kv_win": g["kv_win"], "sink": g["sink"], "o": torch.empty_like(g["q"])})
            del g
        torch.cuda.empty_cache()

        def layer_group(i):
            step(i)
            s, bf = sets[i % n_sets], bufs[i % n_sets]
            for ly in layers:
                dsa.dsa_sparse_attn(ly["q"], ly["kv_win"], s[comp_key], ly["sink"], bf["idx"], scale,
                                    comp_scales=s.get("kv_comp_scale"), out=ly["o"], workspace=bf["workspace"])

        layer_group(0)
        group_launches = dsa.dsa_last_launches()
        torch.cuda.synchronize()
        gg = capture(layer_group, 0, max(1, min(10, 2 * n_sets)))
        gg.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        reps = 3
        for _ in range(reps):
            gg.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        group_ms = e0.elapsed_time(e1) / (reps * max(1, min(10, 2 * n_sets)))
        del gg, layers
        group = {"layers": GROUP_LAYERS, "us": round(group_ms * 1e3, 2),
                 "query_tokens_per_s_per_layer": round(GROUP_LAYERS * w.B * w.S / (group_ms * 1e-3), 1),
                 "speedup_vs_a_step_per_layer": round(GROUP_LAYERS * ms_per_step / group_ms, 3),
                 "reusing_layer_kernels": group_launches[1]}

    # algorithmic work of one attention pass: every valid slot's row once, q, o, idx, sink
    idx_all = torch.stack([bufs[i % n_sets]["idx"] for i in range(n_sets)])
    valid = (idx_all >= 0).view(n_sets, -1).sum(dim=1).double().mean().item()
    esz = 2 if w.dtype == "bf16" else 4
    q_bytes = w.B * w.S * w.H * w.D * esz
    if w.comp_fmt == "fp4":
        # valid window rows are bf16 rows; compressed rows are D/2 nibble bytes + D/16 scale bytes
        win_valid = (idx_all[..., :Wc] >= 0).view(n_sets, -1).sum(dim=1).double().mean().item()
        row_bytes = win_valid * w.D * esz + (valid - win_valid) * (w.D // 2 + w.D // 16)
    else:
        row_bytes = valid * w.D * esz
    attn_bytes = 2 * q_bytes + w.B * w.S * w.L * 4 + w.H * 4 + row_bytes
    # the index part: keys once per batch, index queries and head weights, scores written and read once
    # (MXFP4 index rows: D_I/2 nibble bytes + D_I/32 scale bytes each)
    irow = (w.D_I // 2 + w.D_I // 32) if mx else w.D_I * esz
    index_bytes = (w.B * w.T * irow + w.B * w.S * w.H_I * (irow + esz) + 2 * w.B * w.S * w.T * 4)
    attn_flops = 4.0 * w.H * w.D * valid
    index_flops = 2.0 * w.H_I * w.D_I * visible_pairs(w)
    decode = w.mode == "decode"
    if decode:
        per_launch = attn_bytes + (index_bytes if fused else 0)
        ach = per_launch / (avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(ach / PEAK_HBM_GBS, 4)}
        step_ach = (attn_bytes + index_bytes) / (ms_per_step * 1e-3) / 1e9
        step_roof = {"bound": "hbm", "achieved": round(step_ach, 1), "unit": "GB/s",
                     "frac": round(step_ach / PEAK_HBM_GBS, 4), "algorithmic": attn_bytes + index_bytes}
    else:
        per_launch = attn_flops
        ach = per_launch / (avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(ach / PEAK_BF16_TFLOPS, 4)}
        step_ach = (attn_flops + index_flops) / (ms_per_step * 1e-3) / 1e12
        step_roof = {"bound": "mfma", "achieved": round(step_ach, 1), "unit": "TFLOP/s",
                     "frac": round(step_ach / PEAK_BF16_TFLOPS, 4), "algorithmic": attn_flops + index_flops}
    sha = kernel_src_sha("decode" if decode else "prefill")
    roof["traffic"] = _traffic(w.name, sha)
    roof["kernel"] = dom_names
    roof["avg_launch_us"] = round(avg_ms * 1e3, 2)
    roof["median_launch_us"] = round(med_ms * 1e3, 2)
    roof["launches_timed"] = R
    roof["algorithmic_per_launch"] = per_launch
    entry = {
        "ms_per_step": round(ms_per_step, 5),
        "query_tokens_per_s": round(w.B * w.S / (ms_per_step * 1e-3), 1),
        "launches_per_step": n_launch,
        "kernels": names,
        "roofline": roof,
        "step_roofline": step_roof,
        "rest_of_step_us": None if rest_ms is None else round(rest_ms * 1e3, 2),
        "index_kernel": None if index_ms is None else {
            "us": round(index_ms * 1e3, 2), "algorithmic_bytes": w.B * w.T * irow + w.B * w.S * w.H_I * (irow + esz)
            + w.B * w.S * w.T * 4, "achieved_gbs": round((w.B * w.T * irow + w.B * w.S * w.H_I * (irow + esz)
                                                          + w.B * w.S * w.T * 4) / (index_ms * 1e-3) / 1e9, 1),
            "index_rows": "mxfp4 e2m1 + E8M0/32" if mx else w.dtype},
        "layer_group": group,
        "two_level": two_level,
        "config": {"workload": w.name, "mode": w.mode, "batch": w.B, "query_tokens": w.S, "context": w.end_pos,
                   "heads": w.H, "head_dim": w.D, "window": w.W, "compress_ratio": w.ratio, "index_heads": w.H_I,
                   "index_head_dim": w.D_I, "index_topk": w.index_topk,
                   "compressed_kv": "fp4 e2m1 + E4M3/16" if w.comp_fmt == "fp4" else w.dtype,
                   "index_rows": "mxfp4 e2m1 + E8M0/32" if mx else w.dtype,
                   "input_sets_rotated": n_sets, "kernel_src_sha": sha},
    }
    log(f"[bench] {w.name}: step {ms_per_step * 1e3:.2f} us (wall {wall / a.steps * 1e6:.2f} us), {n_launch} "
        f"launch(es) {names}; dominant {dom_names}: avg {avg_ms * 1e3:.2f} us, median {med_ms * 1e3:.2f} us, "
        f"{roof['achieved']} {roof['unit']} = {roof['frac'] * 100:.1f}% of peak"
        + ("" if rest_ms is None else f"; index+select {rest_ms * 1e3:.2f} us")
        + ("" if group is None else f"; {GROUP_LAYERS}-layer group {group['us']} us "
           f"({group['speedup_vs_a_step_per_layer']}x a step per layer)")
        + ("" if two_level is None else f"; candidate blocks {two_level['candidate_blocks_us']} us, masked index "
           f"{two_level['masked_index_us']} us (full {two_level['full_index_us']} us)"))
    for bf in bufs:
        bf.clear()
    keep = set0
    del sets, bufs
    return entry, keep


# ---------------------------------------------------------------------------- main
def main():
    a = _args()
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); the path shards by batch/query "
              "without collectives and is measured at one GPU's share", file=sys.stderr)
        sys.exit(2)
    if a.calibrate:
        calibrate()
        return
    import torch

    import dsa_synth
    import sparse_mqa_attention_amd as dsa

    def log(msg):
        print(msg, file=sys.stderr, flush=True)

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dsa.dsa_init(dev)
    names = LINE_WORKLOADS if a.workload == "all" else [a.workload]
    headline = HEADLINE if a.workload == "all" else a.workload
    entries = {}
    head_set = None
    for name in names:
        w = dsa_synth.get(name)
        entry, set0 = run_workload(w, a, log)
        entries[name] = entry
        if name == headline:
            head_set = {k: v.cpu() for k, v in set0.items()} if not a.no_cpu_baseline else None
        del set0
        torch.cuda.empty_cache()
    errs = dsa.dsa_device_errors(dev)
    if errs:
        log(f"[bench] device error flags {errs:#x}: a decode rendezvous timed out")
    hw = dsa_synth.get(headline)
    h = entries[headline]
    cpu = None
    if head_set is not None:
        log(f"[bench] CPU oracle baseline on {headline} ({a.cpu_seconds:.0f} s sample)")
        cpu = cpu_baseline(hw, head_set, a.cpu_seconds)
    line = {
        "metric": METRIC,
        "value": h["query_tokens_per_s"],
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": h["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if hw.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": h["config"],
        "roofline": h["roofline"],
        "cpu_baseline": cpu,
        "device_error_flags": errs,
        "workloads": {k: {kk: vv for kk, vv in v.items() if kk != "config"} for k, v in entries.items()},
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
