"""Pins of the sliding-window / attention-sink oracle: special cases with a
known answer, brute force over explicit position lists, invariance to the
excluded positions, the memory formula's printed example, a brute-force
definition of a dead page (no later request length reads it), and the page
release checked against an independent model of it (refcounts, free stack,
-1 marking, a second call, a page shared with the prefix cache, all-or-nothing
failure).  Planted mistakes must fail them."""

import math

import numpy as np
import pytest

import oracle
from oracle import window as W


def data(rng, n, h_q=4, h_kv=2, d=8):
    return (rng.standard_normal((h_q, d)), rng.standard_normal((n, h_kv, d)),
            rng.standard_normal((n, h_kv, d)))


def test_large_window_is_full_attention():
    rng = np.random.default_rng(1)
    q, K, V = data(rng, 37)
    full = oracle.attention_fp64(q, K, V, 0.3)
    for sink, win in ((0, 37), (4, 33), (0, 1000), (37, 1), (10, 27)):
        assert np.allclose(W.attention_window_fp64(q, K, V, 0.3, sink, win), full, atol=1e-14)


def test_window_of_one_is_the_new_token():
    rng = np.random.default_rng(2)
    q, K, V = data(rng, 20)
    got = W.attention_window_fp64(q, K, V, 0.3, 0, 1)
    want = np.repeat(V[-1], 2, axis=0)       # every head of a group reads V[n-1]
    assert np.allclose(got, want, atol=1e-15)


def test_sinks_and_window_bruteforce():
    """Scalar math.exp / math.fsum over an explicitly listed position set."""
    rng = np.random.default_rng(3)
    n, sink, win = 50, 4, 9
    q, K, V = data(rng, n)
    pos = [0, 1, 2, 3] + list(range(41, 50))
    got = W.attention_window_fp64(q, K, V, 0.25, sink, win)
    G = 2
    for h in range(4):
        g = h // G
        s = [0.25 * math.fsum(q[h, i] * K[t, g, i] for i in range(8)) for t in pos]
        m = max(s)
        e = [math.exp(x - m) for x in s]
        den = math.fsum(e)
        for i in range(8):
            want = math.fsum(e[k] * V[pos[k], g, i] for k in range(len(pos))) / den
            assert abs(got[h, i] - want) < 1e-12


def test_excluded_positions_do_not_matter():
    rng = np.random.default_rng(4)
    n, sink, win = 70, 5, 20
    q, K, V = data(rng, n)
    a = W.attention_window_fp64(q, K, V, 0.3, sink, win)
    K2, V2 = K.copy(), V.copy()
    K2[sink:n - win] = 1e3 * rng.standard_normal(K2[sink:n - win].shape)
    V2[sink:n - win] = np.nan
    b = W.attention_window_fp64(q, K2, V2, 0.3, sink, win)
    assert np.array_equal(a, b)


def test_memory_formula_example():
    """The page's example: W = 4096 gives a constant-size cache.  With the
    Llama-3-8B shape (L 32, 8 kv heads x 128 dims, bf16) that is
    2 * 4096 * 32 * 1024 * 2 = 512 MiB per request, with or without growth."""
    assert oracle.sliding_window_bytes(4096, 32, 1024, 2) == 2 * 4096 * 32 * 1024 * 2 == 512 * 2 ** 20
    assert W.window_cache_bytes(4096, 4, 32, 1024, 2) == 2 * 4100 * 32 * 1024 * 2


@pytest.mark.parametrize("sink,win", [(0, 1), (4, 16), (3, 40), (16, 17), (20, 5), (0, 100)])
def test_dead_pages_bruteforce(sink, win):
    """A page is dead at n exactly when no position of it is read at any
    length n' >= n (checked up to n + 200)."""
    for n in range(0, 160):
        dead = set(W.dead_pages(n, sink, win))
        for p in range(-(-n // 16)):
            read_later = any(t in range(16 * p, 16 * p + 16) and t < n2
                             for n2 in range(n, n + 200)
                             for t in W.window_positions(n2, sink, win))
            assert (p in dead) == (not read_later), (n, p)


def test_planted_off_by_one_fails():
    rng = np.random.default_rng(5)
    q, K, V = data(rng, 30)
    orig = W.window_positions
    try:
        W.window_positions = lambda n, s, w: [t for t in range(n) if t < s or t > n - w]
        with pytest.raises(AssertionError):
            test_window_of_one_is_the_new_token()
    finally:
        W.window_positions = orig


# ------------------------------------------------------ window_release pins --
# An independent model of what releasing the dead pages must do, built from
# window_positions alone (never from dead_pages or window_release): a page may
# go back only if no position of it is read at this length or any later one,
# and every such page must go back.  Drops happen request by request, page by
# page; a page returns to the free stack when its last reference is dropped.

def _never_read_again(n, p, sink, win, horizon=200):
    return not any(t < n2 and 16 * p <= t < 16 * p + 16
                   for n2 in range(n, n + horizon)
                   for t in W.window_positions(n2, sink, win))


def _expected_release(rc, free, table, lens, sink, win):
    """(refcounts, free stack top-first, table, released) after the release,
    or None when some drop would hit a page with no reference left."""
    rc, free = dict(rc), list(free)
    table = [list(r) for r in table]
    n_rel = 0
    for b, row in enumerate(table):
        for p in range(-(-lens[b] // 16)):
            if row[p] == -1 or not _never_read_again(lens[b], p, sink, win):
                continue
            blk = row[p]
            if rc.get(blk, 0) <= 0:
                return None
            rc[blk] -= 1
            if rc[blk] == 0:
                free.insert(0, blk)
            row[p] = -1
            n_rel += 1
    return rc, free, table, n_rel


def _scenario(seed, n_req=4, shared_pages=3, cache_refs=True):
    """A pool whose requests share their first `shared_pages` pages (the prefix,
    also referenced once by a prefix cache when cache_refs), then private pages."""
    rng = np.random.default_rng(seed)
    N = 200
    alloc = oracle.RefAllocator(N, rng.permutation(N))
    prefix = [alloc.alloc() for _ in range(shared_pages)]
    lens = [int(rng.integers(16 * shared_pages, 16 * shared_pages + 120)) for _ in range(n_req)]
    table = []
    for b in range(n_req):
        row = list(prefix)
        for blk in prefix:
            alloc.retain(blk)
        while len(row) < -(-lens[b] // 16):
            row.append(alloc.alloc())
        table.append(row)
    if not cache_refs:
        for blk in prefix:
            alloc.release(blk)          # only the tables hold the prefix then
    return alloc, table, lens


def _state(alloc, blocks):
    return {b: alloc.refcount(b) for b in blocks}, alloc.free_list_top_first()


def check_window_release(release):
    """Run `release` (window_release's signature) on seeded scenarios and compare
    with the independent model; raises AssertionError on any difference."""
    for seed in range(6):
        for sink, win in ((0, 1), (4, 16), (3, 40), (16, 17), (20, 5), (0, 30)):
            alloc, table, lens = _scenario(seed, cache_refs=bool(seed % 2))
            blocks = sorted({b for r in table for b in r})
            rc0, free0 = _state(alloc, blocks)
            want = _expected_release(rc0, free0, table, lens, sink, win)
            assert want is not None
            got_n = release(alloc, table, lens, sink, win)
            rc1, free1 = _state(alloc, blocks)
            assert got_n == want[3], (seed, sink, win)
            assert table == want[2], (seed, sink, win)
            assert rc1 == want[0], (seed, sink, win)
            assert free1 == want[1], (seed, sink, win)
            # a second call with the same lengths finds nothing left to drop
            assert release(alloc, table, lens, sink, win) == 0
            assert _state(alloc, blocks) == (rc1, free1)
            # every released page holds no position read at any later length
            for b, row in enumerate(table):
                for p, blk in enumerate(row):
                    if blk == -1:
                        assert _never_read_again(lens[b], p, sink, win)
    # a page mapped by three tables and held by the prefix cache: dropped three
    # times, freed only when the cache lets go as well
    alloc = oracle.RefAllocator(10, list(range(10)))
    blk = alloc.alloc()                       # the cache's reference
    table = []
    for _ in range(3):
        alloc.retain(blk)
        table.append([blk, alloc.alloc(), alloc.alloc()])
    lens = [40, 40, 40]
    assert release(alloc, table, lens, 0, 16) == 3   # page 0 is dead in every request
    assert alloc.refcount(blk) == 1 and blk not in alloc.free_list_top_first()
    assert [r[0] for r in table] == [-1, -1, -1]
    alloc.release(blk)
    assert alloc.free_list_top_first()[0] == blk
    # a dead entry naming a free page: BadBlock, and nothing changes
    alloc = oracle.RefAllocator(10, list(range(10)))
    live = [alloc.alloc() for _ in range(4)]
    alloc.release(live[2])                    # page live[2] is free now
    table = [[live[0], live[1], live[3]], [live[2], live[3], live[1]]]
    for blk in (live[1], live[3]):
        alloc.retain(blk)
    lens = [48, 48]
    before = ([list(r) for r in table], _state(alloc, range(10)))
    with pytest.raises(oracle.BadBlock):
        release(alloc, table, lens, 0, 8)
    assert ([list(r) for r in table], _state(alloc, range(10))) == before


def test_window_release_matches_model():
    check_window_release(W.window_release)


def _planted(kind):
    """window_release with one mistake planted (test of the pins above)."""
    from oracle.allocator import BadBlock

    def release(alloc, table, lens, sink, window, block_size=16):
        n = 0
        for b, row in enumerate(table):
            s = 0 if kind == "sink" else sink
            for p in W.dead_pages(lens[b], s, window, block_size):
                if row[p] == -1:
                    continue
                if kind == "partial" and alloc.refcount(row[p]) == 0:
                    raise BadBlock(row[p])
                alloc.release(row[p])
                if kind != "no_mark":
                    row[p] = -1
                n += 1
        return n
    return release


@pytest.mark.parametrize("kind", ["no_mark", "sink", "partial"])
def test_window_release_planted_mistakes_fail(kind):
    with pytest.raises((AssertionError, oracle.BadBlock)):
        check_window_release(_planted(kind))
