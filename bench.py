"""Benchmark of the sparse MQA attention step on one MI355X.

A step is one pass of the whole path over one batch of synthetic input through
dsa_sparse_attn_step: index scores, index rows (window rows and top-k selection) and sparse
attention.  For decode batches that is one kernel; otherwise the index scores, the index rows and
the attention are three launches (every stage a libdsa kernel).  Inputs are resident in HBM before
timing starts; several input sets are rotated so that the 256 MB Infinity Cache cannot serve one
step from the previous one.

Prints one JSON line (see `--help`).  The roofline object covers the dominant kernel (the decode
kernel that scores, selects and attends, or the sparse attention kernel), timed with HIP events on
the stream it runs on; the CPU baseline is the oracle timed on a bounded sample on the host.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-attn query-tokens/s (decode & prefill) at 1 GPU; % HBM / MFMA peak"
PEAK_HBM_GBS = 8000.0
PEAK_BF16_TFLOPS = 2500.0
ROTATE_BYTES = 768 << 20  # rotate input sets until they span more than the Infinity Cache (256 MB)
# the sources each dominant kernel is compiled from: a change to any of them drops the HBM traffic
# figure taken on the old sources
KERNEL_SOURCES = {
    "decode": ["sparse_mqa_attention_amd/csrc/sparse_attn_decode.hip", "sparse_mqa_attention_amd/csrc/dsa_internal.h",
               "sparse_mqa_attention_amd/csrc/topk_block.h", "sparse_mqa_attention_amd/csrc/index_tile.h"],
    "prefill": ["sparse_mqa_attention_amd/csrc/sparse_attn_prefill_h16.hip",
                "sparse_mqa_attention_amd/csrc/dsa_internal.h"],
}


def _args():
    p = argparse.ArgumentParser(description=__doc__)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=10)
    p.add_argument("--workload", default="decode_b32_ctx8k")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing (profiling runs)")
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    p.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                   help="only run a plain device copy of MIB MiB three times (scale of the HBM byte counters)")
    return p.parse_args()


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

    cores = max(1, min(16, os.cpu_count() or 1))
    comp = (oracle.fp4_rows_decode(cpu_in["kv_comp_fp4"], cpu_in["kv_comp_scale"]) if w.comp_fmt == "fp4"
            else cpu_in["kv_comp"])
    f64 = lambda x: x.float().numpy().astype(np.float64)  # noqa: E731
    _ORACLE_JOB.update(w=w, kv=oracle.kv_concat(cpu_in["kv_win"], comp), win=oracle.window_rows(w.W, 1, w.S,
                       w.start_pos)[0], sink=f64(cpu_in["sink"]), qI=f64(cpu_in["qI"]), kI=f64(cpu_in["kI"]),
                       wt=f64(cpu_in["w"]), q=cpu_in["q"], w_scale=w.D_I ** -0.5 * w.H_I ** -0.5)
    rng = np.random.default_rng(0)
    order = [(b, t) for b in range(w.B) for t in range(w.S)]
    rng.shuffle(order)
    done = 0
    t0 = time.perf_counter()
    with mp.get_context("fork").Pool(cores, initializer=_pool_init) as pool:
        i = 0
        while time.perf_counter() - t0 < target_s and done < 64 * len(order):
            batch = [order[(i + k) % len(order)] for k in range(2 * cores)]
            i += len(batch)
            pool.map(_oracle_query, batch, chunksize=1)
            done += len(batch)
    el = time.perf_counter() - t0
    _ORACLE_JOB.clear()
    return {"value": round(done / el, 2), "unit": "query-tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} queries of {w.name} in random order, each the oracle's scores + top-k + window row "
                      f"+ attention in float64 NumPy, {cores} worker processes x 1 BLAS thread, {el:.1f} s wall"}


# ---------------------------------------------------------------------------- GPU run
def main():
    a = _args()
    if a.copy_calibration:
        copy_calibration(a.copy_calibration)
        return
    if a.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {a.gpus}); the path shards by batch/query "
              "without collectives and is measured at one GPU's share", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import dsa_synth
    import sparse_mqa_attention_amd as dsa

    w = dsa_synth.get(a.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    set0 = dsa_synth.generate(w, seed=0, device=dev)
    set_bytes = sum(dsa_synth.nbytes(t) for t in set0.values())
    n_sets = max(1, min(8, math.ceil(ROTATE_BYTES / set_bytes)))
    sets = [set0] + [dsa_synth.generate(w, seed=s, device=dev) for s in range(1, n_sets)]
    scale = w.D ** -0.5
    w_scale = w.D_I ** -0.5 * w.H_I ** -0.5
    Wc = dsa.dsa_window_cols(w.S, w.start_pos, w.W)
    bufs = []
    for s in sets:
        ws = dsa.dsa_sparse_attn_workspace_size(1 if w.dtype == "bf16" else 0, w.B, w.S, w.H, w.D, w.L)
        bufs.append({"idx": torch.empty(w.B, w.S, Wc + w.K, dtype=torch.int32, device=dev),
                     "scores": torch.empty(w.B, w.S, w.T, dtype=torch.float32, device=dev),
                     "o": torch.empty_like(s["q"]),
                     "workspace": torch.zeros(max(ws, 1), dtype=torch.uint8, device=dev)})
    stream = torch.cuda.current_stream(dev)
    comp_key = "kv_comp_fp4" if w.comp_fmt == "fp4" else "kv_comp"

    # Decode batches the two-phase decode kernel takes score, select and attend inside it (one
    # launch for the whole step); elsewhere the step is index scores, index rows and attention.
    fused = (w.mode == "decode" and w.dtype == "bf16" and w.comp_fmt != "fp4" and w.T <= 2048 and w.D == 512
             and w.H == 64 and w.B * w.S < 256 and w.D_I == 128 and w.H_I <= 64)

    def stage_step(i):
        s, bf = sets[i % n_sets], bufs[i % n_sets]
        dsa.dsa_sparse_attn_step(s["qI"], s["kI"], s["w"], s["q"], s["kv_win"], s[comp_key], s["sink"],
                                 index_topk=w.index_topk, start_pos=w.start_pos, ratio=w.ratio, W=w.W, scale=scale,
                                 w_scale=w_scale, comp_scales=s.get("kv_comp_scale"), out=bf["o"],
                                 scores=bf["scores"], idx=bf["idx"], workspace=bf["workspace"])

    def stage_index(i):
        s, bf = sets[i % n_sets], bufs[i % n_sets]
        dsa.dsa_index_scores(s["qI"], s["kI"], s["w"], w_scale, w.start_pos, w.ratio, out=bf["scores"])

    def stage_select(i):
        s, bf = sets[i % n_sets], bufs[i % n_sets]
        dsa.dsa_select(bf["scores"], w.index_topk, w.start_pos, w.ratio, w.W, w.n_win, out=bf["idx"])

    def stage_attn(i):
        s, bf = sets[i % n_sets], bufs[i % n_sets]
        dsa.dsa_sparse_attn(s["q"], s["kv_win"], s[comp_key], s["sink"], bf["idx"], scale,
                            comp_scales=s.get("kv_comp_scale"), out=bf["o"], workspace=bf["workspace"])

    step = stage_step

    # the dominant kernel and the rest of the step, timed apart
    if fused:
        dominant, rest = stage_step, None
    else:
        dominant = stage_attn

        def rest(i):
            stage_index(i)
            stage_select(i)

    # Steps are captured into HIP graphs of G consecutive steps (rotating input sets), so the
    # timed region measures the GPU, not the host's launch rate.
    G = max(1, min(a.steps, 10))

    def capture(fn, first, count):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for k in range(count):
                fn(first + k)
        return g

    for i in range(min(a.warmup, n_sets)):  # eager warmup: compile-free, initialises every set
        step(i)
    torch.cuda.synchronize()
    full = capture(step, 0, G)
    rem = a.steps % G
    tail = capture(step, 0, rem) if rem else None
    for _ in range(max(1, a.warmup // G)):
        full.replay()
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    t_start.record(stream)
    for _ in range(a.steps // G):
        full.replay()
    if tail is not None:
        tail.replay()
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    gpu_ms = t_start.elapsed_time(t_end)
    ms_per_step = gpu_ms / a.steps

    # the dominant kernel alone: R launches back to back in one graph, bracketed by HIP events
    R = 20
    attn_graph = capture(dominant, 0, R)
    sel_graph = capture(rest, 0, R) if rest is not None else None
    attn_graph.replay()
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record(stream)
    attn_graph.replay()
    e1.record(stream)
    if sel_graph is not None:
        sel_graph.replay()
    e2.record(stream)
    torch.cuda.synchronize()
    attn_avg_ms = e0.elapsed_time(e1) / R
    sel_avg_ms = e1.elapsed_time(e2) / R
    if fused:
        parts = f"index scores+window+top-k+attention (one kernel) {attn_avg_ms * 1e3:.2f} us"
    else:
        parts = f"attention {attn_avg_ms * 1e3:.2f} us, window+index+top-k {sel_avg_ms * 1e3:.2f} us"
    print(f"[bench] {w.name}: step {ms_per_step * 1e3:.2f} us (wall {wall / a.steps * 1e6:.2f} us), {parts}",
          file=sys.stderr)

    # algorithmic work of one sparse-attention launch: every valid slot's row once, q, o, idx, sink
    idx_all = torch.stack([bufs[i % n_sets]["idx"] for i in range(n_sets)])
    valid_per_set = (idx_all >= 0).view(n_sets, -1).sum(dim=1).double().mean().item()
    esz = 2 if w.dtype == "bf16" else 4
    q_bytes = w.B * w.S * w.H * w.D * esz
    if w.comp_fmt == "fp4":
        # valid window rows are bf16 rows; compressed rows are D/2 nibble bytes + D/16 scale bytes
        win_valid = (idx_all[..., :Wc] >= 0).view(n_sets, -1).sum(dim=1).double().mean().item()
        comp_valid = valid_per_set - win_valid
        row_bytes = win_valid * w.D * esz + comp_valid * (w.D // 2 + w.D // 16)
    else:
        row_bytes = valid_per_set * w.D * esz
    alg_bytes = 2 * q_bytes + w.B * w.S * w.L * 4 + w.H * 4 + row_bytes
    if fused:
        # the kernel also reads the index keys, index queries and head weights, and writes each
        # query's scores and reads them back once
        alg_bytes += (w.B * w.T * w.D_I * 2 + w.B * w.S * w.H_I * (w.D_I + 1) * 2 + 2 * w.B * w.S * w.T * 4)
    alg_flops = 4.0 * w.H * w.D * valid_per_set
    if w.mode == "decode":
        achieved = alg_bytes / (attn_avg_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4)}
        per_launch = alg_bytes
    else:
        achieved = alg_flops / (attn_avg_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4)}
        per_launch = alg_flops
    sha = kernel_src_sha(w.mode)
    roof["traffic"] = _traffic(w.name, sha)
    if fused:
        roof["kernel"] = ("dsa_sparse_attn_step (index scores + index rows + gather-attention + split combine, "
                          "one kernel)")
    else:
        roof["kernel"] = "dsa_sparse_attn" + (" (gather-attention + split combine)" if
                                              dsa.dsa_sparse_attn_workspace_size(1, w.B, w.S, w.H, w.D, w.L) else "")
    roof["avg_launch_us"] = round(attn_avg_ms * 1e3, 2)
    roof["algorithmic_per_launch"] = per_launch

    cpu = None
    if not a.no_cpu_baseline:
        cpu_in = {k: v.cpu() for k, v in set0.items()}
        cpu = cpu_baseline(w, cpu_in, a.cpu_seconds)

    queries = w.B * w.S
    line = {
        "metric": METRIC,
        "value": round(queries / (ms_per_step * 1e-3), 1),
        "unit": "query-tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "mode": w.mode, "batch": w.B, "query_tokens": w.S,
                   "context": w.end_pos, "heads": w.H, "head_dim": w.D, "window": w.W, "compress_ratio": w.ratio,
                   "index_heads": w.H_I, "index_head_dim": w.D_I, "index_topk": w.index_topk,
                   "compressed_kv": "fp4 e2m1 + E4M3/16" if w.comp_fmt == "fp4" else w.dtype,
                   "input_sets_rotated": n_sets, "kernel_src_sha": sha},
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
