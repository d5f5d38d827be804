"""Host-side model of the one-wave top-k select (`topk_wave_kernel` in topk.hip).

The kernel's selection steps are restated here in NumPy, bit for bit on the 32-bit keys: the key map
(non-negative float u -> u + 2^31, negative -> -u, so -0.0 meets +0.0), the 8-bit radix passes from
the highest bit where the visible keys differ, the early stop once the chosen digit holds exactly
the keys still to take, and the two emissions: key >= thr in that exact case, keys above tau plus
the first `remaining` keys equal to tau otherwise.  The model checks, on rows built to stress each
branch, that the exact-case threshold keeps the same set as the masked comparison it replaces, that
exactly K positions are kept (the kernel writes one output slot per kept position), and that they
are the K best visible positions with ties to the lower one (DeepSeek V4.1 page, `Indexer.forward`:
top-k by score over the causally visible compressed rows).  The GPU parity tests compare the
kernel itself with the oracle.
"""
import zlib

import numpy as np
import pytest


def _key(u):
    s = np.where(u >> np.uint32(31), np.uint32(0xFFFFFFFF), np.uint32(0)).astype(np.uint32)
    return ((u ^ (s | np.uint32(0x80000000))) - s).astype(np.uint32)


def _select(scores, c, K):
    key = np.zeros(len(scores), np.uint32)
    key[:c] = _key(scores[:c].view(np.uint32))
    kand = int(np.bitwise_and.reduce(key[:c]))
    kor = int(np.bitwise_or.reduce(key[:c]))
    diff = kand ^ kor
    prefix = kand & ~diff & 0xFFFFFFFF
    mask = ~diff & 0xFFFFFFFF
    remaining, exact, lo_end = K, False, 0
    if diff:
        hb = diff.bit_length() - 1
        while True:
            lo = max(hb - 7, 0)
            dmask = ((1 << (hb - lo + 1)) - 1) << lo
            live = (key != 0) & ((key & np.uint32(mask)) == np.uint32(prefix))
            hist = np.bincount(((key[live] & np.uint32(dmask)) >> np.uint32(lo)).astype(np.int64), minlength=256)
            above = 0
            for d in range(255, -1, -1):  # largest digit first
                if above + hist[d] >= remaining:
                    digit, in_digit = d, int(hist[d])
                    break
                above += int(hist[d])
            remaining -= above
            prefix |= digit << lo
            mask |= dmask
            if in_digit == remaining:
                exact, lo_end = True, lo
                break
            if lo == 0:
                break
            hb = lo - 1
    if exact:
        thr = max(prefix & (0xFFFFFFFF << lo_end) & 0xFFFFFFFF, 1)
        keep = np.nonzero(key >= np.uint32(thr))[0]
        masked = np.nonzero((key != 0) & ((key & np.uint32(mask)) >= np.uint32(prefix)))[0]
        assert np.array_equal(keep, masked), "threshold and masked comparison keep different sets"
    else:
        gt = np.nonzero(key > np.uint32(prefix))[0]
        eq = np.nonzero(key == np.uint32(prefix))[0][:remaining]
        keep = np.sort(np.concatenate([gt, eq]))
    return keep, exact


def _best(scores, c, K):
    s = scores[:c].astype(np.float64)
    s = np.where(s == 0.0, 0.0, s)  # -0.0 == +0.0
    return np.sort(np.lexsort((np.arange(c), -s))[:K])


def test_key_map_orders_floats():
    rng = np.random.default_rng(0)
    u = np.concatenate([rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32),
                        np.array([0, 0x80000000, 0x7F800000, 0xFF800000, 1, 0x80000001], np.uint32)])
    f = u.view(np.float32)
    u, f = u[~np.isnan(f)], f[~np.isnan(f)]
    k = _key(u)
    o = np.argsort(f, kind="stable")
    assert np.all(np.diff(k[o].astype(np.int64)) >= 0)
    assert np.array_equal(f[o][1:] == f[o][:-1], k[o][1:] == k[o][:-1])
    assert k.min() >= 1  # 0 stays free for invisible positions
    assert _key(np.array([0x80000000], np.uint32))[0] == _key(np.array([0], np.uint32))[0]


@pytest.mark.parametrize("kind", ["normal", "ties", "zeros", "low_bits", "negative", "near_equal", "equal"])
def test_select_model(kind):
    rng = np.random.default_rng(zlib.crc32(kind.encode()))
    n_exact = 0
    for _ in range(60):
        T = int(rng.integers(600, 2500))
        K = int(rng.integers(1, 600))
        c = int(rng.integers(K + 1, T + 1))
        if kind == "normal":
            s = rng.standard_normal(T).astype(np.float32)
        elif kind == "ties":
            s = rng.integers(-4, 5, T).astype(np.float32)
        elif kind == "zeros":
            s = (rng.integers(0, 2, T) * rng.choice([-1.0, 1.0], T) * 0.0).astype(np.float32)
            s[::7] = rng.standard_normal(len(s[::7]))
        elif kind == "low_bits":  # keys differ only in the last mantissa bits
            s = (1.0 + rng.integers(0, 4, T) * 2.0**-23).astype(np.float32)
        elif kind == "negative":
            s = (-np.abs(rng.standard_normal(T)) * 1e-3).astype(np.float32)
        elif kind == "near_equal":
            s = np.full(T, 2.5, np.float32)
            s[rng.integers(0, T, 5)] = 3.0
        else:  # every visible key equal: no differing bit, no pass
            s = np.full(T, -1.25, np.float32)
        s[c:] = -np.inf
        keep, exact = _select(s, c, K)
        n_exact += exact
        assert len(keep) == K
        assert np.array_equal(keep, _best(s, c, K))
    if kind in ("normal", "negative"):
        assert n_exact > 0  # the exact-case emission is exercised
