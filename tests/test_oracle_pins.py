"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each oracle function is checked against at least one of: a hand-derived
fixture under tests/golden/ (each cites its page and section), a closed form,
brute force on tiny inputs, a library routine for a special case, or an
invariant the definition implies.  The cases are chosen so that a plausible
slip (a dropped ReLU or weight, a transposed operand, an off-by-one in the
visibility, a sink in the numerator, a tie broken the wrong way) fails one.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [ln.strip() for ln in f if ln.strip() and not ln.startswith("#")]


# ---------------------------------------------------------------- window rows
def test_window_rows_golden():
    lines = _lines("window_rows.txt")
    i = 0
    ncases = 0
    while i < len(lines):
        head = lines[i].split()
        assert head[0] == "case"
        W, B, S, sp = map(int, head[1:])
        exp = np.array([list(map(int, lines[i + 1 + t].split())) for t in range(S)])
        got = oracle.window_rows(W, B, S, sp)
        assert got.shape == (B,) + exp.shape
        np.testing.assert_array_equal(got[0], exp)
        i += 1 + S
        ncases += 1
    assert ncases >= 6


def test_window_rows_properties():
    # prefill: every valid entry is a position in [t-W+1, t], each listed once, count min(t+1, W)
    W, S = 16, 64
    r = oracle.window_rows(W, 2, S, 0)
    for t in range(S):
        v = r[1, t][r[1, t] >= 0]
        assert len(set(v.tolist())) == len(v) == min(t + 1, W)
        assert v.min() == max(0, t - W + 1) and v.max() == t
        # -1 only at the tail
        assert np.all(r[1, t][len(v):] == -1)
    # decode: a permutation of the ring once full; slots past start_pos are -1 while filling
    for sp in [1, 5, 127, 128, 129, 8191, 65535]:
        row = oracle.window_rows(128, 1, 1, sp)[0, 0]
        valid = row[row >= 0]
        assert len(set(valid.tolist())) == len(valid) == min(sp + 1, 128)
        assert np.all(valid <= sp)


# ---------------------------------------------------------------- visibility
def test_visible_count_golden():
    for ln in _lines("visible_counts.txt"):
        sp, r, t, c = map(int, ln.split())
        assert int(oracle.visible_count(t, sp, r)) == c


def test_visible_count_brute():
    # group j visible to absolute position p iff all its tokens j*r .. j*r+r-1 are <= p
    for r in [1, 2, 3, 4, 7]:
        for sp in [0, 1, 5, 13]:
            for t in range(20):
                p = sp + t
                brute = sum(1 for j in range(100) if all(tok <= p for tok in range(j * r, j * r + r)))
                assert int(oracle.visible_count(t, sp, r)) == brute


# ---------------------------------------------------------------- fp4 / e4m3
def test_e2m1_golden():
    for ln in _lines("fp4_e2m1.txt"):
        code, val = ln.split()
        got = float(oracle.e2m1_decode(int(code, 16)))
        assert got == float(val) and math.copysign(1, got) == math.copysign(1, float(val))


def test_e4m3_golden_and_library():
    for ln in _lines("e4m3_points.txt"):
        code, val = ln.split()
        got = float(oracle.e4m3_decode(int(code, 16)))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val)
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_decode(np.arange(256))
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(ours[ok], lib[ok])


def test_fp4_packing_and_groups():
    # byte 0x21: element 0 = code 1 (0.5), element 1 = code 2 (1.0); high nibble is the odd element
    packed = np.zeros((1, 16), dtype=np.uint8)  # D = 32 -> 2 groups of 16
    packed[0, 0] = 0x21
    packed[0, 8] = 0xF7  # element 16 = +6, element 17 = -6 (first elements of group 1)
    scales = np.array([[0x38, 0x40]], dtype=np.uint8)  # group 0 scale 1.0, group 1 scale 2.0
    v = oracle.fp4_rows_decode(packed, scales)
    assert v.shape == (1, 32)
    assert v[0, 0] == 0.5 and v[0, 1] == 1.0
    assert v[0, 16] == 12.0 and v[0, 17] == -12.0
    assert np.all(v[0, 2:16] == 0) and np.all(v[0, 18:] == 0)


def test_fp4_decode_against_generator_encoder():
    import dsa_synth

    g = torch.Generator().manual_seed(3)
    x = torch.randn(8, 64, 128, generator=g)
    packed, scales = dsa_synth.encode_fp4_e2m1_e4m3(x, 16)
    dec = oracle.fp4_rows_decode(packed, scales)
    xs = x.double().numpy()
    sc = np.repeat(oracle.e4m3_decode(scales.numpy()), 16, axis=-1)
    # round-to-nearest into e2m1 steps of at most 2 (between 4 and 6): error <= 1 step half-width,
    # plus the saturation when the scale rounded down (|x|/scale may exceed 6 by the scale's rounding)
    err = np.abs(dec - xs)
    assert np.all(err <= sc * 1.0 + np.abs(xs) * 0.07)
    # the decoded magnitudes divided by their scale are e2m1 grid values
    grid = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    ratio = np.abs(dec[sc > 0] / sc[sc > 0])
    assert set(np.unique(ratio).tolist()) <= grid
    # every decoded value is exactly representable in bf16 (dequant-on-load can be exact)
    t = torch.from_numpy(dec)
    assert torch.equal(t.to(torch.bfloat16).double(), t)


def test_fp4_products_exact_in_bf16():
    # all e2m1 x finite-e4m3 products are bf16-exact
    e2 = oracle.e2m1_decode(np.arange(16))
    e4 = oracle.e4m3_decode(np.arange(256))
    e4 = e4[~np.isnan(e4)]
    prod = torch.from_numpy(np.outer(e2, e4))
    assert torch.equal(prod.to(torch.bfloat16).double(), prod)


# ---------------------------------------------------------------- MXFP4 (indexer fp4, E8M0 / 32)
def test_e8m0_golden_and_library():
    for ln in _lines("e8m0_points.txt"):
        code, val = ln.split()
        got = float(oracle.e8m0_decode(int(code, 16)))
        if val == "nan":
            assert math.isnan(got)
        else:
            assert got == float(val)
    # all 256 codes against torch's float8_e8m0fnu conversion
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    lib = codes.view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = oracle.e8m0_decode(np.arange(256))
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(lib))
    ok = ~np.isnan(lib)
    np.testing.assert_array_equal(ours[ok], lib[ok])


def test_mxfp4_packing_and_blocks():
    # D = 64: two blocks of 32 elements, two scale bytes
    packed = np.zeros((1, 32), dtype=np.uint8)
    packed[0, 0] = 0x21   # element 0 = code 1 (0.5), element 1 = code 2 (1.0)
    packed[0, 15] = 0x9F  # element 30 = code 15 (-6), element 31 = code 9 (-0.5): last of block 0
    packed[0, 16] = 0x07  # element 32 = +6: first of block 1
    scales = np.array([[0x7E, 0x81]], dtype=np.uint8)  # block 0 x 0.5, block 1 x 4
    v = oracle.mxfp4_rows_decode(packed, scales)
    assert v.shape == (1, 64)
    assert v[0, 0] == 0.25 and v[0, 1] == 0.5
    assert v[0, 30] == -3.0 and v[0, 31] == -0.25
    assert v[0, 32] == 24.0 and v[0, 33] == 0.0
    assert np.count_nonzero(v) == 5


def test_mxfp4_decode_against_generator_encoder():
    import dsa_synth

    g = torch.Generator().manual_seed(4)
    x = torch.randn(4, 32, 128, generator=g) * torch.exp(torch.randn(4, 32, 1, generator=g))
    x[0, 0, :32] = 0.0  # an all-zero block
    packed, scales = dsa_synth.encode_mxfp4_e8m0(x, 32)
    assert packed.shape == (4, 32, 64) and scales.shape == (4, 32, 4)
    dec = oracle.mxfp4_rows_decode(packed, scales)
    xs = x.double().numpy()
    sc = np.repeat(oracle.e8m0_decode(scales.numpy()), 32, axis=-1)
    # nothing clips (the scale covers the block maximum within the e2m1 range of 6), and rounding
    # to the nearest grid value costs at most half of the widest step (2, between 4 and 6)
    assert np.all(np.abs(xs) <= 6 * sc)
    assert np.all(np.abs(dec - xs) <= 1.0 * sc)
    ratio = np.abs(dec / sc)
    assert set(np.unique(ratio).tolist()) <= {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0}
    assert np.all(dec[0, 0, :32] == 0)
    # values already on a block's grid come back exactly
    again = oracle.mxfp4_rows_decode(*dsa_synth.encode_mxfp4_e8m0(torch.from_numpy(dec).float(), 32))
    np.testing.assert_array_equal(again, dec)
    # every decoded value is exact in bf16 (the page keeps the fake-quantised index keys in bf16)
    t = torch.from_numpy(dec)
    assert torch.equal(t.to(torch.bfloat16).double(), t)


def test_mxfp4_index_scores_brute():
    """Scores on MXFP4 index inputs: a scalar loop that decodes every element from the golden
    e2m1 and E8M0 tables itself equals the oracle's decode followed by its score definition."""
    import dsa_synth

    e2m1 = {int(c, 16): float(v) for c, v in (ln.split() for ln in _lines("fp4_e2m1.txt"))}
    g = torch.Generator().manual_seed(9)
    B, S, T, H, D = 1, 3, 5, 2, 64
    qp, qs = dsa_synth.encode_mxfp4_e8m0(torch.randn(B, S, H, D, generator=g), 32)
    kp, ks = dsa_synth.encode_mxfp4_e8m0(torch.randn(B, T, D, generator=g) * 4, 32)
    w = torch.randn(B, S, H, generator=g).double().numpy()
    sp, ratio, ws = 7, 2, 0.3
    got = oracle.index_scores(oracle.mxfp4_rows_decode(qp, qs), oracle.mxfp4_rows_decode(kp, ks), w, ws, sp, ratio)

    def elem(packed, scales, idx, d):
        byte = int(packed[idx + (d // 2,)])
        code = byte & 0xF if d % 2 == 0 else byte >> 4
        return e2m1[code] * 2.0 ** (int(scales[idx + (d // 32,)]) - 127)

    qpn, qsn, kpn, ksn = qp.numpy(), qs.numpy(), kp.numpy(), ks.numpy()
    for t in range(S):
        c = (sp + t + 1) // ratio
        for j in range(T):
            if j >= c:
                assert got[0, t, j] == -np.inf
                continue
            tot = 0.0
            for h in range(H):
                dot = sum(elem(qpn, qsn, (0, t, h), d) * elem(kpn, ksn, (0, j), d) for d in range(D))
                tot += w[0, t, h] * max(dot, 0.0)
            assert abs(got[0, t, j] - ws * tot) <= 1e-12 * max(1.0, abs(ws * tot))


# ---------------------------------------------------------------- candidate blocks (two-level selection)
def test_candidate_blocks_hand_golden():
    lines = _lines("candidate_blocks_hand.txt")
    row = np.array([float(x) for x in lines[0].split()[1:]])
    for ln in lines[1:]:
        lhs, rhs = ln.split("->")
        c, n = map(int, lhs.split())
        want = [int(x) for x in rhs.split()]
        got = np.nonzero(oracle.candidate_blocks_row(row, c, n, 4))[0].tolist()
        assert got == want, (c, n, got, want)


def _blocks_brute(row, c, n, bs):
    blocks = []
    for i in range((c + bs - 1) // bs):
        m = -math.inf
        for j in range(i * bs, min((i + 1) * bs, c)):
            m = max(m, row[j])
        blocks.append((-m, i))
    blocks.sort()
    return sorted(i for _, i in blocks[:n])


@pytest.mark.parametrize("seed", range(6))
def test_candidate_blocks_brute_and_invariants(seed):
    rng = np.random.default_rng(seed)
    T, bs = 61, 4
    for _ in range(60):
        row = rng.integers(-3, 4, size=T).astype(np.float64) if seed % 2 else rng.standard_normal(T)
        c = int(rng.integers(0, T + 1))
        n = int(rng.integers(1, 20))
        got = oracle.candidate_blocks_row(row, c, n, bs)
        assert np.nonzero(got)[0].tolist() == _blocks_brute(row.tolist(), c, n, bs)
        cb = -(-c // bs)
        assert got.sum() == min(n, cb)
    # the mask: every visible position when all visible blocks fit; positions of chosen blocks only
    S, sp, ratio = 5, 30, 2
    scores = rng.standard_normal((2, S, T))
    m_all = oracle.candidate_mask(scores, sp, ratio, 100, bs)
    c = oracle.visible_count(np.arange(S), sp, ratio)
    for t in range(S):
        assert np.array_equal(m_all[:, t], np.broadcast_to(np.arange(T) < min(T, c[t]), (2, T)))
    m = oracle.candidate_mask(scores, sp, ratio, 3, bs)
    assert np.all(m.reshape(2, S, -1).sum(-1) <= 3 * bs)
    # the top-k of masked scores lies inside the candidates when they hold at least K positions
    masked = np.where(m, scores, -np.inf)
    sel = oracle.topk_select(masked, 6, sp, ratio, 0)
    for b in range(2):
        for t in range(S):
            picked = sel[b, t][sel[b, t] >= 0]
            assert np.all(m[b, t, picked])


def test_planted_candidate_slip_is_caught(monkeypatch):
    """A block scored by its sum instead of its maximum breaks the hand-worked example."""
    import oracle.dsa_oracle as od

    monkeypatch.setattr(od, "candidate_blocks_row", _sum_blocks)
    monkeypatch.setattr(oracle, "candidate_blocks_row", _sum_blocks)
    with pytest.raises(AssertionError):
        test_candidate_blocks_hand_golden()


def _sum_blocks(row, c, n, bs):
    nblk = -(-len(row) // bs)
    cb = -(-c // bs)
    sums = np.array([row[i * bs:min((i + 1) * bs, c)].sum() for i in range(cb)])
    out = np.zeros(nblk, dtype=bool)
    if cb:
        pick = oracle.topk_select_row(sums, min(n, cb), cb, 0)
        out[pick[pick >= 0]] = True
    return out


# ---------------------------------------------------------------- index scores
def test_index_scores_hand_golden():
    d = {ln.split()[0]: ln.split()[1:] for ln in _lines("index_scores_hand.txt")}
    q = np.array(list(map(float, d["q"]))).reshape(2, 2)
    k = np.array(list(map(float, d["k"]))).reshape(3, 2)
    w = np.array(list(map(float, d["w"])))
    S = 3
    qI = np.broadcast_to(q, (1, S, 2, 2)).copy()
    wt = np.broadcast_to(w, (1, S, 2)).copy()
    got = oracle.index_scores(qI, k[None], wt, 1.0, start_pos=0, ratio=1)
    for t in range(S):
        exp = np.array([float(x) for x in d[f"t{t}"]])
        np.testing.assert_array_equal(got[0, t], exp)


def _scores_brute(qI, kI, w, w_scale, start_pos, ratio):
    B, S, H, Dd = qI.shape
    T = kI.shape[1]
    out = np.zeros((B, S, T))
    for b in range(B):
        for t in range(S):
            c = (start_pos + t + 1) // ratio
            for j in range(T):
                if j >= c:
                    out[b, t, j] = -math.inf
                    continue
                acc = 0.0
                for h in range(H):
                    dot = 0.0
                    for e in range(Dd):
                        dot += float(qI[b, t, h, e]) * float(kI[b, j, e])
                    acc += float(w[b, t, h]) * (dot if dot > 0 else 0.0)
                out[b, t, j] = w_scale * acc
    return out


@pytest.mark.parametrize("start_pos,S,ratio", [(0, 9, 2), (0, 8, 4), (11, 1, 4), (6, 1, 1)])
def test_index_scores_brute(start_pos, S, ratio):
    rng = np.random.default_rng(start_pos * 31 + S)
    B, H, Dd = 2, 3, 5
    T = (start_pos + S) // ratio
    qI = rng.standard_normal((B, S, H, Dd))
    kI = rng.standard_normal((B, T, Dd))
    w = rng.standard_normal((B, S, H)) * 0.5
    got = oracle.index_scores(qI, kI, w, 0.37, start_pos, ratio)
    exp = _scores_brute(qI, kI, w, 0.37, start_pos, ratio)
    np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-12)
    rows = [(b, t) for b in range(B) for t in range(S)]
    got_rows = oracle.index_scores_rows(qI, kI, w, 0.37, start_pos, ratio, rows)
    np.testing.assert_allclose(got_rows, exp.reshape(B * S, T), rtol=1e-12, atol=1e-12)


def test_index_scores_invariants():
    rng = np.random.default_rng(7)
    B, S, H, Dd, T = 1, 1, 4, 8, 6
    qI = rng.standard_normal((B, S, H, Dd))
    kI = rng.standard_normal((B, T, Dd))
    w = rng.standard_normal((B, S, H))
    base = oracle.index_scores(qI, kI, w, 1.0, start_pos=T - 1, ratio=1)
    # positive scaling of w scales scores; permuting heads with their weights changes nothing
    np.testing.assert_allclose(oracle.index_scores(qI, kI, 3 * w, 1.0, T - 1, 1), 3 * base, rtol=1e-12)
    perm = rng.permutation(H)
    np.testing.assert_allclose(oracle.index_scores(qI[:, :, perm], kI, w[:, :, perm], 1.0, T - 1, 1), base,
                               rtol=1e-12)
    # rectification: negating every query head with positive weights flips which heads count
    wpos = np.abs(w)
    s_pos = oracle.index_scores(qI, kI, wpos, 1.0, T - 1, 1)
    s_neg = oracle.index_scores(-qI, kI, wpos, 1.0, T - 1, 1)
    dots = np.einsum("hd,td->ht", qI[0, 0], kI[0])
    np.testing.assert_allclose(s_pos - s_neg, (wpos[0, 0] @ dots)[None, None], rtol=1e-12, atol=1e-12)
    assert np.all(s_pos >= 0) and np.all(s_neg >= 0)


# ---------------------------------------------------------------- top-k
def _parse_topk(ln):
    a, b, c = ln.split("|")
    scores = np.array([float(x) for x in a.split()])
    K, cnt, off = map(int, b.split())
    exp = np.array(list(map(int, c.split())))
    return scores, K, cnt, off, exp


def test_topk_hand_golden():
    for ln in _lines("topk_hand.txt"):
        scores, K, c, off, exp = _parse_topk(ln)
        got = oracle.topk_select_row(scores, K, c, off)
        np.testing.assert_array_equal(got, exp, err_msg=ln)


def _topk_brute(s, K, c, off):
    order = sorted(range(c), key=lambda j: (-s[j], j))
    chosen = sorted(order[: min(K, c)])
    return [j + off for j in chosen] + [-1] * (K - min(K, c))


def test_topk_brute_force_sort():
    rng = np.random.default_rng(11)
    for trial in range(400):
        T = int(rng.integers(1, 24))
        s = rng.integers(-3, 4, size=T).astype(np.float64)  # many ties
        if trial % 3 == 0:
            s = rng.standard_normal(T)
        K = int(rng.integers(1, T + 1))
        c = int(rng.integers(0, T + 1))
        off = int(rng.integers(0, 50))
        got = oracle.topk_select_row(s, K, c, off).tolist()
        assert got == _topk_brute(s.tolist(), K, c, off), (s, K, c, off)


def test_topk_full_matrix_and_invariants():
    rng = np.random.default_rng(5)
    B, S, T, ratio = 2, 40, 10, 4
    scores = rng.standard_normal((B, S, T))
    c = oracle.visible_count(np.arange(S), 0, ratio)
    scores[:, np.arange(T)[None, :] >= c[:, None]] = -np.inf
    idx = oracle.topk_select(scores, 6, 0, ratio, offset=100)
    assert idx.shape == (B, S, 6)
    for b in range(B):
        for t in range(S):
            row = idx[b, t]
            n = min(6, int(c[t]))
            assert np.all(row[n:] == -1) and np.all(row[:n] >= 100)
            assert np.all(np.diff(row[:n]) > 0)
            assert np.all(row[:n] < 100 + c[t])
            if c[t] <= 6:
                np.testing.assert_array_equal(row[:n], 100 + np.arange(n))


# ---------------------------------------------------------------- attention
def test_attention_hand_closed_form():
    q = np.array([[[[1.0, 0.0]]]])  # B=S=H=1, D=2
    kv = np.array([[[2.0, 0.0], [0.0, 1.0]]])
    idx = np.array([[[0, 1]]])
    o = oracle.sparse_attn(q, kv, np.array([0.0]), idx, 1.0)
    e2 = math.exp(2.0)
    np.testing.assert_allclose(o[0, 0, 0], [2 * e2 / (e2 + 2), 1 / (e2 + 2)], rtol=1e-14)


def _dense_with_sink(q, kv, sink, idx, scale):
    """Dense attention over all n rows with non-selected rows masked, plus one
    extra logit column for the sink whose value vector is zero; duplicates in
    an index row count with their multiplicity (log of the count added)."""
    from scipy.special import softmax

    B, S, H, D = q.shape
    n = kv.shape[1]
    out = np.zeros((B, S, H, D))
    for b in range(B):
        for t in range(S):
            mult = np.zeros(n)
            for j in idx[b, t]:
                if j >= 0:
                    mult[j] += 1
            with np.errstate(divide="ignore"):
                logm = np.where(mult > 0, np.log(mult), -np.inf)
            logits = scale * q[b, t] @ kv[b].T + logm[None, :]  # [H, n]
            full = np.concatenate([logits, sink[:, None]], axis=1)
            p = softmax(full, axis=1)
            vals = np.concatenate([kv[b], np.zeros((1, D))], axis=0)
            out[b, t] = p @ vals
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attention_vs_dense_masked(seed):
    rng = np.random.default_rng(seed)
    B, S, H, D, n, L = 2, 3, 4, 8, 12, 7
    q = rng.standard_normal((B, S, H, D))
    kv = rng.standard_normal((B, n, D))
    sink = rng.standard_normal(H)
    idx = rng.integers(-1, n, size=(B, S, L))
    idx[0, 0, :] = -1  # an all-invalid row
    idx[1, 2, 1] = idx[1, 2, 0] = 5  # a duplicate
    got = oracle.sparse_attn(q, kv, sink, idx, 0.3)
    exp = _dense_with_sink(q, kv, sink, idx, 0.3)
    np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-14)
    assert np.all(got[0, 0] == 0)


def test_attention_sdpa_when_sink_vanishes():
    # with the sink logit far below every logit the sink term drops out, and the result is
    # plain softmax attention over the gathered rows: torch's scaled_dot_product_attention
    rng = np.random.default_rng(9)
    H, D, n = 4, 16, 10
    q = rng.standard_normal((1, 1, H, D))
    kv = rng.standard_normal((1, n, D))
    idx = np.array([[[3, 1, 7, 0, 9]]])
    got = oracle.sparse_attn(q, kv, np.full(H, -1e4), idx, D ** -0.5)
    rows = torch.from_numpy(kv[0, idx[0, 0]])  # [5, D]
    qt = torch.from_numpy(q[0, 0])[:, None, :]  # [H, 1, D]
    ref = torch.nn.functional.scaled_dot_product_attention(qt, rows.expand(H, -1, -1), rows.expand(H, -1, -1))
    np.testing.assert_allclose(got[0, 0], ref[:, 0].numpy(), rtol=1e-12, atol=1e-14)


def test_attention_closed_forms():
    rng = np.random.default_rng(4)
    H, D, n = 3, 6, 5
    q = rng.standard_normal((1, 1, H, D))
    kv = rng.standard_normal((1, n, D))
    sink = rng.standard_normal(H)
    sc = 0.7
    # one valid slot: o = row * e^l / (e^l + e^sink)
    o = oracle.sparse_attn(q, kv, sink, np.array([[[-1, 2, -1]]]), sc)
    for h in range(H):
        lg = sc * float(q[0, 0, h] @ kv[0, 2])
        np.testing.assert_allclose(o[0, 0, h], kv[0, 2] / (1 + math.exp(sink[h] - lg)), rtol=1e-13)
    # m identical rows listed: o = row * m e^l / (m e^l + e^sink)
    o = oracle.sparse_attn(q, kv, sink, np.array([[[4, 4, 4, -1]]]), sc)
    for h in range(H):
        lg = sc * float(q[0, 0, h] @ kv[0, 4])
        np.testing.assert_allclose(o[0, 0, h], kv[0, 4] * 3 / (3 + math.exp(sink[h] - lg)), rtol=1e-13)
    # order inside an index row does not matter
    a = oracle.sparse_attn(q, kv, sink, np.array([[[0, 3, 1, -1, 4]]]), sc)
    b = oracle.sparse_attn(q, kv, sink, np.array([[[4, -1, 1, 0, 3]]]), sc)
    np.testing.assert_allclose(a, b, rtol=1e-13)
    # a huge sink drives the output to zero without NaN; a tiny one leaves plain softmax weights
    o = oracle.sparse_attn(q, kv, np.full(H, 1e4), np.array([[[0, 1]]]), sc)
    assert np.all(np.isfinite(o)) and np.all(np.abs(o) < 1e-100)


def test_attention_rows_and_concat():
    rng = np.random.default_rng(8)
    B, S, H, D = 2, 4, 2, 4
    q = rng.standard_normal((B, S, H, D))
    win = rng.standard_normal((B, 3, D))
    comp = rng.standard_normal((B, 5, D))
    kv = oracle.kv_concat(win, comp)
    assert kv.shape == (B, 8, D)
    np.testing.assert_array_equal(kv[:, 3:], comp)
    idx = rng.integers(-1, 8, size=(B, S, 5))
    full = oracle.sparse_attn(q, kv, np.zeros(H), idx, 0.5)
    rows = [(1, 2), (0, 0), (1, 3)]
    part = oracle.sparse_attn_rows(q, kv, np.zeros(H), idx, 0.5, rows)
    for n, (b, t) in enumerate(rows):
        np.testing.assert_array_equal(part[n], full[b, t])


# ---------------------------------------------------------------- planted slips
def test_planted_slips_are_caught(monkeypatch):
    """Plant plausible mistakes in the oracle (on the CPU) and check a pin fails."""
    import oracle.dsa_oracle as od

    d = {ln.split()[0]: ln.split()[1:] for ln in _lines("index_scores_hand.txt")}
    q = np.array(list(map(float, d["q"]))).reshape(2, 2)
    k = np.array(list(map(float, d["k"]))).reshape(3, 2)
    w = np.array(list(map(float, d["w"])))
    exp = np.array([float(x) for x in d["t2"]])

    def score_t2():
        return od.index_scores(q[None, None], k[None], w[None, None], 1.0, start_pos=2, ratio=1)[0, 0]

    np.testing.assert_array_equal(score_t2(), exp)
    # dropped ReLU
    monkeypatch.setattr(od.np, "maximum", lambda a, b: a)
    assert not np.array_equal(score_t2(), exp)
    monkeypatch.undo()
    # transposed operand (key dims reversed)
    kk = k[:, ::-1].copy()
    assert not np.array_equal(od.index_scores(q[None, None], kk[None], w[None, None], 1.0, 2, 1)[0, 0], exp)
    # sink in the numerator too would break the closed form with one slot
    e2 = math.exp(2.0)
    o = od.sparse_attn(np.array([[[[1.0, 0.0]]]]), np.array([[[2.0, 0.0], [0.0, 1.0]]]), np.array([0.0]),
                       np.array([[[0, 1]]]), 1.0)
    assert not np.allclose(o[0, 0, 0], [2 * e2 / (e2 + 1), 1 / (e2 + 1)])
    # ties to the higher index would fail the brute-force sort on "5 5 5 5 | 2 4 0 | 0 1"
    s = np.array([5.0, 5.0, 5.0, 5.0])
    assert od.topk_select_row(s, 2, 4, 0).tolist() == [0, 1]
    assert _topk_brute(s.tolist(), 2, 4, 0) == [0, 1]


def test_planted_mxfp4_slips_are_caught(monkeypatch):
    """Plausible mistakes in the MXFP4 decode (nibble order swapped, a block of 16 instead of 32,
    a bias of 128) each break a pin."""
    import oracle.dsa_oracle as od

    test_mxfp4_packing_and_blocks()
    real = od.mxfp4_rows_decode

    def swapped(packed, scales, block=32):
        p = np.asarray(packed, dtype=np.int64)
        return real(((p & 0xF) << 4) | (p >> 4), scales, block)

    def block16(packed, scales, block=32):  # the compressed KV's group size with the indexer's scales
        sc = np.asarray(scales)
        return real(packed, np.concatenate([sc, sc], axis=-1), 16)

    for slip in (swapped, block16):
        monkeypatch.setattr(od, "mxfp4_rows_decode", slip)
        monkeypatch.setattr(oracle, "mxfp4_rows_decode", slip)
        with pytest.raises(AssertionError):
            test_mxfp4_packing_and_blocks()
        monkeypatch.undo()
    monkeypatch.setattr(od.np, "ldexp", lambda m, e: m * 2.0 ** (np.asarray(e) - 1))
    with pytest.raises(AssertionError):
        test_e8m0_golden_and_library()
    monkeypatch.undo()


# ---------------------------------------------------------------- output epilogue and cache write
def test_bf16_rne_against_torch():
    rng = np.random.default_rng(11)
    x = (rng.standard_normal(20000) * np.exp(rng.standard_normal(20000) * 8)).astype(np.float32)
    # exact ties: a bf16 value plus half of its last place, for even and odd last bits
    base = torch.randn(2000).to(torch.bfloat16).float().numpy()
    half = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, half, np.array([0.0, -0.0, np.inf, -np.inf], dtype=np.float32)])
    lib = torch.from_numpy(x).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(oracle.bf16_rne(x), lib)
    assert np.isnan(oracle.bf16_rne(np.array([np.nan], dtype=np.float32))[0])


def test_e4m3_rne_against_torch():
    rng = np.random.default_rng(12)
    v = np.abs(rng.standard_normal(20000) * np.exp(rng.uniform(-9, 6, 20000))).astype(np.float32)
    v = v[v <= 448]
    # exact ties between neighbouring E4M3 values, subnormal and normal
    grid = np.unique(oracle.e4m3_decode(np.arange(0, 0x7F)))
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    v = np.concatenate([v, mids, np.array([0.0, 2.0 ** -10, 2.0 ** -9, 448.0], dtype=np.float32)])
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).double().numpy()
    np.testing.assert_array_equal(oracle.e4m3_rne(v), lib)
    # reading: past the largest finite value the scale saturates at 448 (torch gives NaN)
    assert oracle.e4m3_rne(np.array([500.0, 1e6], dtype=np.float32)).tolist() == [448.0, 448.0]


def test_rope_rotate_complex_and_inverse():
    rng = np.random.default_rng(13)
    S, H, D, P = 6, 4, 24, 5
    x = rng.standard_normal((2, S, H, D))
    ang = rng.standard_normal((S, P)) * 4
    freqs = np.stack([np.cos(ang), np.sin(ang)], -1)
    y = oracle.rope_rotate(x, freqs)
    np.testing.assert_array_equal(y[..., : D - 2 * P], x[..., : D - 2 * P])  # leading dims untouched
    z = x[..., D - 2 * P:].reshape(2, S, H, P, 2)
    zc = (z[..., 0] + 1j * z[..., 1]) * np.exp(1j * ang)[None, :, None, :]
    np.testing.assert_allclose(y[..., D - 2 * P::2], zc.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y[..., D - 2 * P + 1::2], zc.imag, rtol=0, atol=1e-13)
    np.testing.assert_allclose(oracle.rope_rotate(y, freqs, inverse=True), x, rtol=0, atol=1e-13)


def test_rope_rotate_bf16_against_torch_complex():
    """The page's rotation of a bf16 view: complex64 product, written back as bf16."""
    rng = np.random.default_rng(14)
    S, H, D, P = 7, 3, 64, 16
    x = torch.randn(S, H, D).to(torch.bfloat16)
    ang = (rng.standard_normal((S, P)) * 3).astype(np.float32)
    freqs = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    ours = oracle.rope_rotate_bf16(x.float().numpy(), freqs)
    xc = torch.view_as_complex(x[..., -2 * P:].float().unflatten(-1, (-1, 2)).contiguous())
    fc = torch.complex(torch.from_numpy(freqs[..., 0]), torch.from_numpy(freqs[..., 1]))[:, None, :]
    lib = torch.view_as_real(xc * fc).flatten(-2).to(torch.bfloat16).float().numpy()
    np.testing.assert_array_equal(ours[..., -2 * P:], lib)
    np.testing.assert_array_equal(ours[..., : D - 2 * P], x[..., : D - 2 * P].float().numpy())


def test_fp4_quantiser_against_generator_encoder():
    """The oracle's fp4/E4M3 quantiser (numpy, float32 steps) and the generator's encoder (torch)
    are independent codings of one rule: the same bytes."""
    import dsa_synth

    g = torch.Generator().manual_seed(15)
    x = torch.randn(6, 33, 512, generator=g) * torch.exp(torch.randn(6, 33, 1, generator=g) * 2)
    x[0, 0, :16] = 0.0
    p1, s1 = dsa_synth.encode_fp4_e2m1_e4m3(x, 16)
    p2, s2 = oracle.fp4_quant_e4m3_g16(x.numpy())
    np.testing.assert_array_equal(p2, p1.numpy())
    np.testing.assert_array_equal(s2, s1.numpy())
    # decoding gives values within the widest half step (1 x scale) of the input, or past the largest
    # e2m1 value when the scale rounded down; a zero scale only for blocks whose amax/6 rounds to 0
    dec = oracle.fp4_rows_decode(p2, s2)
    sc = np.repeat(oracle.e4m3_decode(s2), 16, axis=-1)
    xs = x.double().numpy()
    pos = sc > 0
    assert np.all(np.abs(dec - xs)[pos] <= np.maximum(sc, np.abs(xs) - 6 * sc)[pos])
    assert np.all(np.abs(xs[~pos]) < 6 * 2.0 ** -10)


def test_compress_kv_write_composition():
    rng = np.random.default_rng(16)
    B, n, D, rd = 2, 5, 64, 16
    lat = torch.randn(B, n, D).to(torch.bfloat16).float().numpy()
    ang = (rng.standard_normal((n, rd // 2)) * 3).astype(np.float32)
    freqs = np.stack([np.cos(ang), np.sin(ang)], -1).astype(np.float32)
    packed, scales = oracle.compress_kv_write(lat, freqs, rd)
    assert packed.shape == (B, n, D // 2) and scales.shape == (B, n, D // 16)
    rot = oracle.rope_rotate_bf16(lat[:, :, None, :], freqs)[:, :, 0, :]
    p2, s2 = oracle.fp4_quant_e4m3_g16(rot)
    np.testing.assert_array_equal(packed, p2)
    np.testing.assert_array_equal(scales, s2)
    # the first D - rd dims are quantised unrotated
    p3, _ = oracle.fp4_quant_e4m3_g16(lat)
    np.testing.assert_array_equal(packed[..., : (D - rd) // 2], p3[..., : (D - rd) // 2])
