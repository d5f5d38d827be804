"""CPU oracle of the sparse MQA attention step -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module.  The product path (the HIP library and its binding) never
calls it and shares no code with it.

Everything is computed in float64 from the exact input values (bf16, fp32,
e2m1 and E4M3 all decode exactly into float64), with no blocking, fusion or
reordering beyond what the definitions state.  Citations name the DeepSeek V4.1
model pages by the class or function that holds the step:

* window rows      -- `get_window_topk_idxs` (page "attention/attend/selected")
* index scores     -- `Indexer.forward`: per-head dot of the index query with the
                      shared index key, rectified, weighted by `weights_proj`
                      times index_head_dim**-0.5 * index_n_heads**-0.5, summed
                      over heads
* visibility       -- `Indexer.forward`: a compressed group becomes visible once
                      the query has passed its last token
* top-k selection  -- `Indexer.forward`: top-k by score, re-sorted into position
                      order, unreachable -> -1, the rest shifted by `offset`
* attention        -- `sparse_attn_kernel` / `sparse_attn`: gather the indexed
                      rows of the one shared KV tensor (key = value), softmax over
                      the valid slots with the per-head sink logit added to the
                      denominator only, -1 slots ignored, all-invalid rows -> 0
* fp4 compressed KV -- `_compress_kv` (page "reindex-layer/read-weights"): e2m1
                      values with one E4M3 scale per 16 elements
* candidate blocks  -- `Indexer.forward` with a candidate source: the source layer
                      picks `candidate_topk_blocks` blocks of `candidate_block_size`
                      compressed positions from its scores (`select_candidate_blocks`,
                      body not on the pages), and later indexers mask their scores to
                      -inf outside those blocks before their own top-k
* output epilogue   -- `Attention.forward`: the inverse rotary embedding on the last
                      rope_head_dim dims of o, at the query's position
* cache write       -- `_compress_kv`: rotary embedding of the latent's last
                      rope_head_dim dims at the group's position, fp4 with E4M3 scales
                      per 16, written into the compressed cache
* MXFP4 index q/k   -- `Indexer.forward` quantises the index queries and keys to
                      fp4, and `_compress_kv` states the indexer's blocks: 32
                      elements per E8M0 (power-of-two) scale.  The scores are the
                      same definition over the decoded values.

Readings where the pages leave a step open (each also listed with the design
notes): a candidate block's score is the largest visible score in it, a block
is visible when any of its positions is, and the chosen blocks are the
`candidate_topk_blocks` best visible blocks, ties to the lower block; ties in
the top-k go to the lower position; scores are exact (not the
eager bf16 rounding of the page's einsum); visibility uses the single formula
c(t) = (start_pos + t + 1) // ratio, which reproduces both of the page's
branches (prefill from 0, one-token decode).

Parity pins: every function here is checked in `tests/test_oracle_pins.py`
against hand-derived fixtures, closed forms, brute force or library routines.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "visible_count",
    "window_rows",
    "index_scores",
    "index_scores_rows",
    "topk_select",
    "topk_select_row",
    "candidate_blocks_row",
    "candidate_mask",
    "e2m1_decode",
    "e4m3_decode",
    "fp4_rows_decode",
    "e8m0_decode",
    "rope_rotate",
    "bf16_rne",
    "e4m3_rne",
    "rope_rotate_bf16",
    "fp4_quant_e4m3_g16",
    "compress_kv_write",
    "mxfp4_rows_decode",
    "kv_concat",
    "sparse_attn",
    "sparse_attn_rows",
]


# ----------------------------------------------------------------------------
# visibility and window rows
# ----------------------------------------------------------------------------
def visible_count(t, start_pos: int, ratio: int):
    """Compressed rows visible to query t: floor((start_pos + t + 1) / ratio).

    `Indexer.forward`: group j covers tokens j*ratio .. j*ratio+ratio-1 and is
    visible once the query's absolute position p = start_pos + t has reached
    its last token, i.e. j*ratio + ratio - 1 <= p.  In prefill (start_pos 0)
    this is the page's (t+1)//ratio; in one-token decode it is end_pos//ratio.
    """
    t = np.asarray(t, dtype=np.int64)
    return (start_pos + t + 1) // ratio


def window_rows(W: int, B: int, S: int, start_pos: int) -> np.ndarray:
    """Window index rows of `get_window_topk_idxs`, int64 [B, S, Wc].

    Prefill (start_pos == 0): query t lists the chunk positions of its causal
    window, starting at max(0, t - W + 1), min(S, W) slots, -1 for slots past t.
    Decode (start_pos > 0, one query): the W ring slots oldest first, i.e.
    slot (start_pos mod W) + 1 ... W - 1, then 0 ... start_pos mod W, with -1
    for slots whose position has not been written yet (slot > start_pos).
    """
    if start_pos == 0:
        n = min(S, W)
        rows = np.empty((S, n), dtype=np.int64)
        for t in range(S):
            first = max(0, t - W + 1)
            for s in range(n):
                pos = first + s
                rows[t, s] = pos if pos <= t else -1
    else:
        if S != 1:
            raise ValueError("the page's decode branch lists one query's ring (S must be 1)")
        oldest = start_pos % W + 1
        slots = list(range(oldest, W)) + list(range(0, oldest))
        rows = np.array([[s if s <= start_pos else -1 for s in slots]], dtype=np.int64)
    return np.broadcast_to(rows, (B,) + rows.shape).copy()


# ----------------------------------------------------------------------------
# index scores
# ----------------------------------------------------------------------------
def _f64(x) -> np.ndarray:
    if hasattr(x, "detach"):  # torch tensor: exact widening through float32
        x = x.detach().cpu().float().numpy()
    return np.asarray(x, dtype=np.float64)


def index_scores(qI, kI, w, w_scale: float, start_pos: int, ratio: int) -> np.ndarray:
    """I[b,t,j] = w_scale * sum_h w[b,t,h] * max(0, sum_d qI[b,t,h,d] kI[b,j,d]).

    `Indexer.forward`: einsum "bshd,btd->bsht" of the index query heads with the
    one shared key per compressed row, ReLU, times the head weights, summed over
    heads.  Entries with j >= c(t) (not yet visible) are -inf, as the page's
    masked_fill does.  Shapes: qI [B,S,H_I,D_I], kI [B,T,D_I], w [B,S,H_I];
    returns float64 [B,S,T].
    """
    q = _f64(qI)
    k = _f64(kI)
    wt = _f64(w)
    B, S, H, Dd = q.shape
    T = k.shape[1]
    dots = np.einsum("bshd,btd->bsht", q, k)  # exact products, fp64 sums
    out = float(w_scale) * np.einsum("bsh,bsht->bst", wt, np.maximum(dots, 0.0))
    c = visible_count(np.arange(S), start_pos, ratio)
    invisible = np.arange(T)[None, :] >= c[:, None]  # [S,T]
    out[:, invisible] = -np.inf
    return out


def index_scores_rows(qI, kI, w, w_scale: float, start_pos: int, ratio: int, rows) -> np.ndarray:
    """`index_scores` for a list of (b, t) query rows only: float64 [len(rows), T]."""
    k = _f64(kI)
    T = k.shape[1]
    out = np.empty((len(rows), T), dtype=np.float64)
    for n, (b, t) in enumerate(rows):
        q = _f64(qI[b, t])  # [H_I, D_I]
        wt = _f64(w[b, t])  # [H_I]
        dots = q @ k[b].T  # [H_I, T]
        out[n] = float(w_scale) * (wt @ np.maximum(dots, 0.0))
        c = int(visible_count(t, start_pos, ratio))
        out[n, c:] = -np.inf
    return out


# ----------------------------------------------------------------------------
# top-k selection
# ----------------------------------------------------------------------------
def topk_select_row(scores_row: np.ndarray, K: int, c: int, offset: int) -> np.ndarray:
    """One query's index row: int64 [K].

    `Indexer.forward`: among the c visible positions keep the min(K, c) best
    scores, ties to the lower position (reading: the page's topk leaves tie
    order open), list them in ascending position order, add `offset`, and fill
    the rest of the K slots with -1 (the page's sort-then-mask leaves the -1
    entries at the tail).

    Selection by value threshold: tau is the n-th largest visible score; every
    position scoring above tau is kept, and of those scoring exactly tau the
    lowest positions are kept until n are chosen.
    """
    out = np.full(K, -1, dtype=np.int64)
    n = min(K, c)
    if n == 0:
        return out
    s = np.asarray(scores_row[:c], dtype=np.float64)
    tau = np.sort(s)[::-1][n - 1]
    above = s > tau
    at = s == tau
    need = n - int(above.sum())
    keep = above | (at & (np.cumsum(at) <= need))
    chosen = np.nonzero(keep)[0]
    assert chosen.size == n
    out[:n] = chosen + offset
    return out


def topk_select(scores: np.ndarray, index_topk: int, start_pos: int, ratio: int, offset: int) -> np.ndarray:
    """Index rows for all queries: int64 [B, S, K] with K = min(index_topk, T).

    K is one number for the whole call (`Indexer.forward` takes
    min(index_topk, end_pos // ratio)), so early prefill rows carry a -1 tail.
    """
    B, S, T = scores.shape
    K = min(index_topk, T)
    out = np.empty((B, S, K), dtype=np.int64)
    c = visible_count(np.arange(S), start_pos, ratio)
    for b in range(B):
        for t in range(S):
            out[b, t] = topk_select_row(scores[b, t], K, int(c[t]), offset)
    return out


# ----------------------------------------------------------------------------
# two-level selection: candidate blocks of the source layer
# ----------------------------------------------------------------------------
def candidate_blocks_row(scores_row: np.ndarray, c: int, n_blocks: int, block_size: int) -> np.ndarray:
    """Chosen blocks of one query (`select_candidate_blocks`, reading): bool [ceil(T/block_size)].

    Block i covers compressed positions i*block_size .. +block_size-1 and is
    visible when its first position is (i*block_size < c).  Its score is the
    largest of its visible scores.  The min(n_blocks, visible blocks) best
    visible blocks are chosen, equal scores going to the lower block (the same
    rule as the top-k, applied to blocks).
    """
    s = np.asarray(scores_row, dtype=np.float64)
    nblk = -(-s.shape[0] // block_size)
    cb = -(-c // block_size)  # visible blocks
    bs = np.array([s[i * block_size:min((i + 1) * block_size, c)].max() for i in range(cb)])
    chosen = np.zeros(nblk, dtype=bool)
    if cb == 0:
        return chosen
    pick = topk_select_row(bs, min(n_blocks, cb), cb, 0)
    chosen[pick[pick >= 0]] = True
    return chosen


def candidate_mask(scores: np.ndarray, start_pos: int, ratio: int, n_blocks: int, block_size: int) -> np.ndarray:
    """Per-position candidate mask bool [B, S, T] of the source layer's scores: position j of query
    t is a candidate when its block is chosen (invisible positions are never candidates)."""
    B, S, T = scores.shape
    c = visible_count(np.arange(S), start_pos, ratio)
    out = np.zeros((B, S, T), dtype=bool)
    for b in range(B):
        for t in range(S):
            ct = int(min(T, c[t]))
            blk = candidate_blocks_row(scores[b, t], ct, n_blocks, block_size)
            out[b, t] = np.repeat(blk, block_size)[:T] & (np.arange(T) < ct)
    return out


# ----------------------------------------------------------------------------
# fp4 e2m1 with E4M3 group scales
# ----------------------------------------------------------------------------
def e2m1_decode(code) -> np.ndarray:
    """FP4 E2M1 (OCP Microscaling spec): sign bit 3, 2 exponent bits (bias 1),
    1 mantissa bit; exponent 0 is subnormal (0 or 0.5)."""
    c = np.asarray(code, dtype=np.int64) & 0xF
    sign = np.where(c & 0x8, -1.0, 1.0)
    e = (c >> 1) & 0x3
    m = c & 0x1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return sign * mag


def e4m3_decode(code) -> np.ndarray:
    """FP8 E4M3FN (OCP 8-bit floating point spec): sign bit 7, 4 exponent bits
    (bias 7), 3 mantissa bits; exponent 0 is subnormal; S.1111.111 is NaN; no
    infinities."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def fp4_rows_decode(packed, scales, group: int = 16) -> np.ndarray:
    """Compressed KV rows from packed nibbles [..., D/2] and E4M3 scales [..., D/group].

    `_compress_kv`: groups of 16 elements share one E4M3 scale; element 2k is the
    low nibble of byte k, element 2k+1 the high nibble (the generator's packing).
    value = e2m1(nibble) * e4m3(scale of its group).
    """
    p = np.asarray(packed.cpu().numpy() if hasattr(packed, "cpu") else packed, dtype=np.int64)
    sc = np.asarray(scales.cpu().numpy() if hasattr(scales, "cpu") else scales, dtype=np.int64)
    lo = e2m1_decode(p & 0xF)
    hi = e2m1_decode(p >> 4)
    vals = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    vals[..., 0::2] = lo
    vals[..., 1::2] = hi
    s = np.repeat(e4m3_decode(sc), group, axis=-1)
    return vals * s


# ----------------------------------------------------------------------------
# MXFP4: e2m1 with E8M0 block scales (the indexer's format)
# ----------------------------------------------------------------------------
def e8m0_decode(code) -> np.ndarray:
    """E8M0 scale (OCP Microscaling spec): an unsigned 8-bit biased exponent, value
    2**(code - 127); code 255 is NaN.  No sign, no mantissa."""
    c = np.asarray(code, dtype=np.int64) & 0xFF
    return np.where(c == 255, np.nan, np.ldexp(1.0, c - 127))


def mxfp4_rows_decode(packed, scales, block: int = 32) -> np.ndarray:
    """Index rows from packed e2m1 nibbles [..., D/2] and E8M0 scales [..., D/block].

    `_compress_kv` / `Indexer.forward`: blocks of 32 consecutive elements share one
    E8M0 scale; element 2k is the low nibble of byte k, element 2k+1 the high
    nibble.  value = e2m1(nibble) * 2**(scale - 127).
    """
    p = np.asarray(packed.cpu().numpy() if hasattr(packed, "cpu") else packed, dtype=np.int64)
    sc = np.asarray(scales.cpu().numpy() if hasattr(scales, "cpu") else scales, dtype=np.int64)
    vals = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    vals[..., 0::2] = e2m1_decode(p & 0xF)
    vals[..., 1::2] = e2m1_decode(p >> 4)
    return vals * np.repeat(e8m0_decode(sc), block, axis=-1)


# ----------------------------------------------------------------------------
# rotary embedding and the compressed-cache write
# ----------------------------------------------------------------------------
def rope_rotate(x, freqs, inverse: bool = False) -> np.ndarray:
    """Rotary embedding of the last 2*P dims of x [..., S, H, D] by freqs [S, P, 2] (cos, sin) of
    each row's position (`apply_rotary_emb`, body not on the pages; reading: dims 2i, 2i+1 of the
    rotated part are the real and imaginary parts of one complex number, multiplied by
    cos + i sin, or by its conjugate for the inverse).  Exact, float64."""
    x = np.array(x, dtype=np.float64)
    f = np.asarray(freqs, dtype=np.float64)
    P = f.shape[-2]
    cos = f[..., 0][:, None, :]  # [S, 1, P]: the same angle for every head
    sin = f[..., 1][:, None, :]
    if inverse:
        sin = -sin
    a = x[..., -2 * P::2].copy()
    b = x[..., -2 * P + 1::2].copy()
    x[..., -2 * P::2] = a * cos - b * sin
    x[..., -2 * P + 1::2] = a * sin + b * cos
    return x


def bf16_rne(x) -> np.ndarray:
    """float32 values rounded to bfloat16, to nearest with ties to even (returned as float32)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    out = (r & 0xFFFFFFFF).astype(np.uint32).view(np.float32)
    return np.where(nan, np.float32(np.nan), out)


def e4m3_rne(x) -> np.ndarray:
    """Non-negative float32 values rounded to the nearest FP8 E4M3 value, ties to the even code,
    saturating at 448 (reading: a scale past the largest E4M3 value would otherwise be NaN).
    Returned as float64 (exact)."""
    v = np.asarray(x, dtype=np.float64)
    e = np.floor(np.log2(np.where(v > 0, v, 1.0)))
    e = np.clip(e, -6, 8)                     # subnormals share the step of exponent -6
    step = np.ldexp(1.0, (e - 3).astype(np.int64))  # 3 mantissa bits
    q = v / step                              # exact: a power-of-two division
    r = np.floor(q)
    frac = q - r
    r = np.where((frac > 0.5) | ((frac == 0.5) & (np.mod(r, 2) == 1)), r + 1, r)
    return np.minimum(r * step, 448.0)


_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def rope_rotate_bf16(x_bf16, freqs) -> np.ndarray:
    """The page's rotation of a bf16 tensor (`apply_rotary_emb` on a bf16 view): float32 products and
    sums (no fused multiply-add), rounded back to bf16.  x [..., S, H, D] as float values, freqs
    [S, P, 2] float32.  Returns float32 values that are bf16."""
    x = np.array(x_bf16, dtype=np.float32)
    f = np.asarray(freqs, dtype=np.float32)
    P = f.shape[-2]
    cos = f[..., 0][:, None, :]
    sin = f[..., 1][:, None, :]
    a = x[..., -2 * P::2].copy()
    b = x[..., -2 * P + 1::2].copy()
    re = np.float32(a * cos) - np.float32(b * sin)
    im = np.float32(a * sin) + np.float32(b * cos)
    x[..., -2 * P::2] = bf16_rne(re)
    x[..., -2 * P + 1::2] = bf16_rne(im)
    return x


def fp4_quant_e4m3_g16(x) -> tuple:
    """fp4 e2m1 with one E4M3 scale per 16 consecutive elements (`_compress_kv`: groups of 16 with
    E4M3 scales; the quantiser's body is not on the pages).  Reading, each step in float32 as a
    kernel would take it: scale = E4M3(amax / 6); code = the e2m1 value nearest x / scale (ties to
    the even code, 6 at most, sign kept); a zero scale gives zero codes.  Returns (packed uint8
    [..., D/2] with element 2k in the low nibble of byte k, scale codes uint8 [..., D/16])."""
    x = np.asarray(x, dtype=np.float32)
    g = x.reshape(*x.shape[:-1], x.shape[-1] // 16, 16)
    amax = np.abs(g).max(axis=-1)
    scale = e4m3_rne(np.float32(amax) / np.float32(6.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = np.where(scale[..., None] > 0, g / scale[..., None], np.float32(0.0)).astype(np.float32)
    m = np.abs(y).astype(np.float64)
    code = np.zeros(m.shape, dtype=np.int64)
    for i in range(7):
        mid = 0.5 * (_E2M1_MAG[i] + _E2M1_MAG[i + 1])
        code += (m > mid) | ((m == mid) & ((i + 1) % 2 == 0))
    code = np.minimum(code, 7) | np.where(y < 0, 8, 0)
    code = code.reshape(x.shape).astype(np.uint8)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    # scale codes: E4M3 bit patterns of the (non-negative) scale values
    sc = _e4m3_code(scale.astype(np.float64))
    return packed, sc


def _e4m3_code(v) -> np.ndarray:
    """E4M3 code of non-negative values on the E4M3 grid."""
    v = np.asarray(v, dtype=np.float64)
    e = np.floor(np.log2(np.where(v > 0, v, 1.0))).astype(np.int64)
    normal = v >= 2.0 ** -6
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, v / np.ldexp(1.0, e) - 1.0, v / 2.0 ** -6) * 8
    code = (exp_field << 3) | np.rint(mant).astype(np.int64)
    return np.where(v > 0, code, 0).astype(np.uint8)


def compress_kv_write(latent_bf16, freqs, rope_dim: int) -> tuple:
    """`_compress_kv` after the compressor: the latent rows [B, n, D] (bf16 values) rotated on their
    last rope_dim dims by freqs [n, rope_dim/2, 2] of each group's position (in the page's precision),
    then fp4 with E4M3 scales per 16.  Returns (packed [B, n, D/2], scales [B, n, D/16])."""
    x = np.asarray(latent_bf16, dtype=np.float32)
    rot = rope_rotate_bf16(x[:, :, None, :], freqs)[:, :, 0, :]  # one 'head'
    return fp4_quant_e4m3_g16(rot)


# ----------------------------------------------------------------------------
# sparse attention
# ----------------------------------------------------------------------------
def kv_concat(kv_win, kv_comp) -> np.ndarray:
    """The one KV tensor attention indexes: window rows, then compressed rows.

    `Attention.forward` concatenates the window KV and the compressed KV along
    the row axis and shifts the compressed indices by the window row count.
    """
    a = _f64(kv_win)
    if kv_comp is None:
        return a
    c = kv_comp if isinstance(kv_comp, np.ndarray) else _f64(kv_comp)
    return np.concatenate([a, np.asarray(c, dtype=np.float64)], axis=1)


def _attend_one(qbt: np.ndarray, kvb: np.ndarray, sink: np.ndarray, idx_row: np.ndarray, scale: float):
    """One query: qbt [H, D], kvb [n, D], sink [H], idx_row [L] -> [H, D]."""
    idx_row = np.asarray(idx_row, dtype=np.int64)
    assert np.all((idx_row == -1) | ((idx_row >= 0) & (idx_row < kvb.shape[0]))), "index out of range"
    valid = idx_row[idx_row >= 0]
    H, D = qbt.shape
    if valid.size == 0:
        return np.zeros((H, D), dtype=np.float64)
    rows = kvb[valid]  # every slot counts on its own, duplicates included
    logits = scale * (qbt @ rows.T)  # [H, nv]
    m = np.maximum(logits.max(axis=1), sink)  # [H]
    e = np.exp(logits - m[:, None])
    den = e.sum(axis=1) + np.exp(sink - m)
    return (e @ rows) / den[:, None]


def sparse_attn(q, kv, sink, idx, scale: float) -> np.ndarray:
    """o[b,t,h] = sum_s e^{l_s} kv[idx_s] / (sum_s e^{l_s} + e^{sink_h}).

    `sparse_attn_kernel`: l_s = scale * q[b,t,h] . kv[b, idx[b,t,s]] over the
    slots with idx != -1; the key and the value are the same row; the sink
    logit (unscaled) joins the denominator only; a row with no valid slot
    gives 0.  q [B,S,H,D], kv [B,n,D], sink [H], idx [B,S,L] -> float64 [B,S,H,D].
    """
    qq = _f64(q)
    kvv = kv if isinstance(kv, np.ndarray) else _f64(kv)
    sk = _f64(sink)
    ii = np.asarray(idx.cpu().numpy() if hasattr(idx, "cpu") else idx, dtype=np.int64)
    B, S, H, D = qq.shape
    out = np.empty((B, S, H, D), dtype=np.float64)
    for b in range(B):
        for t in range(S):
            out[b, t] = _attend_one(qq[b, t], kvv[b], sk, ii[b, t], scale)
    return out


def sparse_attn_rows(q, kv, sink, idx, scale: float, rows) -> np.ndarray:
    """`sparse_attn` for a list of (b, t) query rows only: float64 [len(rows), H, D]."""
    kvv = kv if isinstance(kv, np.ndarray) else _f64(kv)
    sk = _f64(sink)
    out = []
    for b, t in rows:
        qbt = _f64(q[b, t])
        ir = np.asarray(idx[b, t].cpu().numpy() if hasattr(idx, "cpu") else idx[b, t], dtype=np.int64)
        out.append(_attend_one(qbt, kvv[b], sk, ir, scale))
    return np.stack(out) if out else np.zeros((0,) + tuple(q.shape[2:]))
