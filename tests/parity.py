"""Parity rules shared by the GPU tests (test infrastructure; compares HIP results with the oracle).

Top-k rows: the -1 count and position are exact; rows that see at most K positions are exact;
rows whose K-th and (K+1)-th oracle scores differ by more than 1e-3 relative must select the
exact oracle set; the remaining rows may differ only inside the band around the K-th score.
Attention outputs: max |gpu - oracle| <= 2e-2 (bf16) or 1e-5 (fp32).
"""
from __future__ import annotations

import numpy as np

import dsa_synth
import oracle

ATTN_TOL = {"bf16": 2e-2, "f32": 1e-5}
GAP_REL = 1e-3


def sample_rows(w: dsa_synth.Workload, n_random: int = 6, seed: int = 1):
    """(b, t) rows for sampled checks: the first queries, the c(t) = K crossover, the last ones."""
    rng = np.random.default_rng(seed)
    ts = {0, 1, 2, 3, w.S // 2, w.S - 2, w.S - 1}
    cross = w.K * w.ratio - 1 - w.start_pos  # first query with c(t) = K
    for d in (-2, -1, 0, 1, 2):
        ts.add(cross + d)
    ts = sorted(t for t in ts if 0 <= t < w.S)
    rows = [(b, t) for b in sorted({0, w.B - 1}) for t in ts]
    for _ in range(n_random):
        rows.append((int(rng.integers(0, w.B)), int(rng.integers(0, w.S))))
    return sorted(set(rows))


def check_topk_row(got: np.ndarray, scores_row: np.ndarray, K: int, c: int, offset: int, ctx: str = "") -> str:
    """Validate one index row against oracle scores (float64, length >= c). Returns the rule used."""
    got = np.asarray(got, dtype=np.int64)
    n = min(K, c)
    assert got.shape == (K,), ctx
    assert np.all(got[n:] == -1), f"{ctx}: -1 tail wrong (n={n}) {got[max(0, n - 3):n + 3]}"
    sel = got[:n]
    assert np.all(sel >= offset) and np.all(sel < offset + c), f"{ctx}: index out of visible range"
    assert np.all(np.diff(sel) > 0), f"{ctx}: not strictly ascending"
    if c <= K:
        assert np.array_equal(sel, offset + np.arange(c)), f"{ctx}: c<=K row must be 0..c-1"
        return "exact"
    s = np.asarray(scores_row[:c], dtype=np.float64)
    order = np.sort(s)[::-1]
    sk, sk1 = order[K - 1], order[K]
    denom = max(abs(sk), abs(sk1))
    rel = (sk - sk1) / denom if denom > 0 else 0.0
    ref = oracle.topk_select_row(s, K, c, offset)
    if rel > GAP_REL:
        assert np.array_equal(np.sort(sel), ref[:n]), f"{ctx}: set differs with gap {rel:.2e}"
        return "set"
    delta = GAP_REL * denom
    chosen = sel - offset
    assert np.all(s[chosen] >= sk - delta), f"{ctx}: selected score below the band"
    mask = np.ones(c, dtype=bool)
    mask[chosen] = False
    assert np.all(s[mask] <= sk + delta), f"{ctx}: unselected score above the band"
    return "banded"


def max_abs_err(a, b) -> float:
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def score_bound(qI: np.ndarray, kI: np.ndarray, w: np.ndarray, w_scale: float) -> np.ndarray:
    """Float32-accumulation error bound scale for index scores: w_scale * sum_h |w| sum_d |q k|.

    qI [S,H,D], kI [T,D], w [S,H] -> [S,T]."""
    return abs(w_scale) * np.einsum("sh,sht->st", np.abs(w), np.einsum("shd,td->sht", np.abs(qI), np.abs(kI)))
