"""Pins of the prefix-cache and copy-on-write oracle against formulations
other than its own: whole-prefix tuples instead of chained page keys,
reference-count conservation, a hand-worked eviction order, and the
properties copy-on-write must give.  Planted mistakes in the oracle must fail
these pins."""

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle.prefix_cache import RefPrefixCache, reserve_cow

BS = 16


WORDS = [[w * 100 + i for i in range(BS)] for w in range(3)]


def prompt(rng, pages, vocab=3, tail=0):
    """Whole pages drawn from three fixed page contents (so prompts share
    prefixes, and the same page content follows different prefixes), then
    `tail` loose tokens."""
    toks = []
    for _ in range(pages):
        toks += WORDS[int(rng.integers(0, vocab))]
    return toks + [int(x) for x in rng.integers(0, 1000, tail)]


def brute_match_len(inserted, tenant, tokens):
    """Longest m such that every prefix of k <= m whole pages was inserted for
    this tenant (the definition, as sets of full prefixes)."""
    m = 0
    while (m + 1) * BS <= len(tokens) and (tenant, tuple(tokens[:(m + 1) * BS])) in inserted:
        m += 1
    return m


def run_without_eviction(seed, planted=None):
    rng = np.random.default_rng(seed)
    alloc = oracle.RefAllocator(400)
    cache = RefPrefixCache(alloc)
    if planted:
        planted(cache)
    inserted = {}   # (tenant, prefix tuple) -> page holding that prefix's last page
    held = []       # pages mapped by requests
    for _ in range(40):
        tenant = int(rng.integers(0, 2))
        toks = prompt(rng, int(rng.integers(0, 5)), tail=int(rng.integers(0, 16)))
        got = cache.match(tenant, toks)
        m = brute_match_len(inserted, tenant, toks)
        assert len(got) == m
        for k, blk in enumerate(got):
            assert blk == inserted[(tenant, tuple(toks[:(k + 1) * BS]))]
        # the request computes the rest of its whole pages into fresh pages
        row = list(got) + [alloc.alloc() for _ in range(len(toks) // BS - m)]
        held.extend(got)
        held.extend(row[m:])
        cache.insert(tenant, toks, row)
        for k in range(len(toks) // BS):
            inserted.setdefault((tenant, tuple(toks[:(k + 1) * BS])), row[k])
    return alloc, cache, held


@pytest.mark.parametrize("seed", range(6))
def test_match_is_longest_inserted_prefix(seed):
    alloc, cache, held = run_without_eviction(seed)
    # conservation: every reference is a request mapping or a cache entry
    total = sum(alloc.refcount(b) for b in range(alloc.num_blocks))
    assert total == len(held) + cache.num_entries()
    assert alloc.num_free() + len({*held} | {e["block"] for e in cache.entries.values()}) == alloc.num_blocks


def test_tenants_never_share():
    alloc = oracle.RefAllocator(20)
    cache = RefPrefixCache(alloc)
    toks = list(range(40))
    row = [alloc.alloc() for _ in range(2)]
    assert cache.insert(7, toks, row) == 2
    assert cache.match(8, toks) == []
    assert cache.match(7, toks) == row
    assert cache.match(7, toks[:31]) == row[:1]      # one whole page only


def test_page_reused_only_after_identical_prefix():
    alloc = oracle.RefAllocator(20)
    cache = RefPrefixCache(alloc)
    a = [1] * 16 + [2] * 16
    b = [3] * 16 + [2] * 16          # same second page, different first page
    cache.insert(0, a, [alloc.alloc(), alloc.alloc()])
    assert cache.match(0, b) == []


def test_eviction_order_worked_example():
    """Hand-worked: pages p0 <- p1 (a chain) and q0, all inserted, then
    touched in the order p-chain, q0.  Nothing is evictable while a request
    maps it; once released, leaves go oldest first and a parent becomes
    evictable after its child."""
    alloc = oracle.RefAllocator(10, initial_free_order=list(range(10)))
    cache = RefPrefixCache(alloc)
    p = [5] * 32
    q = [6] * 16
    rp = [alloc.alloc(), alloc.alloc()]      # pages 0, 1
    rq = [alloc.alloc()]                     # page 2
    cache.insert(0, p, rp)                   # ticks 1 (p0), 2 (p1)
    cache.insert(0, q, rq)                   # tick 3 (q0)
    assert [alloc.refcount(b) for b in (0, 1, 2)] == [2, 2, 2]
    assert cache.evict(5) == []              # the requests still map them
    for b in rp + rq:
        alloc.release(b)
    # candidates: p1 (leaf, tick 2) and q0 (tick 3); p0 has a child
    assert cache.evict(1) == [1]
    # now p0 (tick 1) is a leaf and older than q0 (tick 3)
    assert cache.evict(5) == [0, 2]
    assert cache.num_entries() == 0 and alloc.num_free() == 10
    # a freed page is handed out next (LIFO): the last one freed is on top
    assert alloc.alloc() == 2


def test_match_touch_changes_eviction_order():
    alloc = oracle.RefAllocator(10, initial_free_order=list(range(10)))
    cache = RefPrefixCache(alloc)
    a, b = [1] * 16, [2] * 16
    ra, rb = [alloc.alloc()], [alloc.alloc()]    # pages 0 and 1
    cache.insert(0, a, ra)
    cache.insert(0, b, rb)
    alloc.release(0), alloc.release(1)
    got = cache.match(0, a)                      # touches page 0 last
    alloc.release(got[0])
    assert cache.evict(1) == [1]


# ---------------------------------------------------------- copy on write --
def test_reserve_cow_properties():
    rng = np.random.default_rng(3)
    alloc = oracle.RefAllocator(64, initial_free_order=rng.permutation(64))
    # a parent of 37 tokens forked into three children (shared pages)
    parent = [alloc.alloc() for _ in range(3)]
    table = [list(parent)]
    for _ in range(3):
        for blk in parent:
            alloc.retain(blk)
        table.append(list(parent))
    lens = [37] * 4
    before = [list(r) for r in table]
    slots, copies = reserve_cow(alloc, table, lens, [0, 1, 5, 20])
    # the parent appends nothing and is untouched
    assert table[0] == before[0] and lens[0] == 37
    # each writing child got its own copy of the shared partial last page
    assert [c[0] for c in copies] == [parent[2]] * 3
    news = [c[1] for c in copies]
    assert len(set(news)) == 3 and not set(news) & set(parent)
    for child, new in zip(table[1:], news):
        assert child[2] == new and child[:2] == parent[:2]
    assert alloc.refcount(parent[2]) == 1            # only the parent maps it now
    # every written slot lies in a page mapped once
    for s in slots:
        assert alloc.refcount(s // BS) == 1
    assert lens == [37, 38, 42, 57]
    assert len(slots) == 26


def test_reserve_cow_rolls_back():
    alloc = oracle.RefAllocator(5, initial_free_order=list(range(5)))
    shared = [alloc.alloc()]
    alloc.retain(shared[0])
    table = [list(shared), list(shared)]
    lens = [3, 3]
    state = (list(alloc._stack), list(alloc._rc))
    with pytest.raises(oracle.NoBlocks):
        reserve_cow(alloc, table, lens, [1, 100])
    assert (list(alloc._stack), list(alloc._rc)) == state
    assert table == [shared, shared] and lens == [3, 3]


# ---------------------------------------------------------- planted mistakes --
def _no_tenant(cache):
    orig = cache._keys
    cache._keys = lambda tenant, tokens: [(0,) + k[1:] for k in orig(0, tokens)]


def _no_parent(cache):
    bs = cache.bs
    cache._keys = lambda tenant, tokens: [
        (int(tenant), None, tuple(int(t) for t in tokens[i * bs:(i + 1) * bs]))
        for i in range(len(tokens) // bs)]


def test_planted_mistakes_fail_the_pins():
    with pytest.raises(AssertionError):
        for seed in range(6):
            run_without_eviction(seed, planted=_no_parent)
    alloc = oracle.RefAllocator(20)
    cache = RefPrefixCache(alloc)
    _no_tenant(cache)
    toks = list(range(32))
    cache.insert(7, toks, [alloc.alloc(), alloc.alloc()])
    assert cache.match(8, toks) != []      # the tenant pin would catch this


@settings(max_examples=40, deadline=None)
@given(seed=st.integers(0, 2 ** 31 - 1), n_ops=st.integers(1, 60))
def test_random_ops_keep_references_consistent(seed, n_ops):
    """Matches, inserts, request retirements and evictions in any order: no
    page is freed while mapped, and every reference is accounted for."""
    rng = np.random.default_rng(seed)
    alloc = oracle.RefAllocator(60, initial_free_order=rng.permutation(60))
    cache = RefPrefixCache(alloc)
    live = []
    for _ in range(n_ops):
        op = rng.integers(0, 3)
        if op == 0:
            tenant = int(rng.integers(0, 2))
            toks = prompt(rng, int(rng.integers(1, 4)))
            got = cache.match(tenant, toks)
            new = []
            try:
                for _ in range(len(toks) // BS - len(got)):
                    new.append(alloc.alloc())
            except oracle.NoBlocks:
                for b in got + new:
                    alloc.release(b)
                continue
            row = got + new
            cache.insert(tenant, toks, row)
            live.append(row)
        elif op == 1 and live:
            for b in live.pop(int(rng.integers(0, len(live)))):
                alloc.release(b)
        else:
            freed = cache.evict(int(rng.integers(1, 4)))
            mapped = {b for r in live for b in r}
            assert not set(freed) & mapped
        total = sum(alloc.refcount(b) for b in range(60))
        assert total == sum(len(r) for r in live) + cache.num_entries()


def test_copy_pages_duplicates_and_touches_nothing_else():
    """The oracle's page copy: each destination page ends up byte-equal to
    its source in every layer (K, V and the 8-bit scales); every other page
    is unchanged; out-of-range and self pairs are skipped; a request read
    through the copy sees exactly what it saw through the shared page."""
    rng = np.random.default_rng(11)
    for dtype in ("bf16", "fp8"):
        L, N, H, D = 2, 9, 2, 64
        pool = oracle.RefPool(L, N, H, D, 16, dtype)
        pool.K = rng.integers(0, 255, pool.K.shape).astype(pool.K.dtype)
        pool.V = rng.integers(0, 255, pool.V.shape).astype(pool.V.dtype)
        if dtype == "fp8":
            pool.Ks = rng.random(pool.Ks.shape).astype(np.float32) + 0.5
            pool.Vs = rng.random(pool.Vs.shape).astype(np.float32) + 0.5
        before = pool.K.copy(), pool.V.copy()
        src, dst = [3, 0, 42, 5], [7, 2, 1, 5]        # 42: out of range; 5 -> 5: itself
        table_shared = np.array([4, 3], np.int32)     # a request whose second page is 3
        k0, v0 = pool.gather_raw(1, table_shared, 30)
        pool.copy_pages(src, dst)
        for s_, d_ in ((3, 7), (0, 2)):
            assert np.array_equal(pool.K[:, d_], pool.K[:, s_]) and np.array_equal(pool.V[:, d_], pool.V[:, s_])
            if dtype == "fp8":
                assert np.array_equal(pool.Ks[:, d_], pool.Ks[:, s_])
        untouched = [b for b in range(N) if b not in (7, 2)]
        assert np.array_equal(pool.K[:, untouched], before[0][:, untouched])
        assert np.array_equal(pool.V[:, untouched], before[1][:, untouched])
        k1, v1 = pool.gather_raw(1, np.array([4, 7], np.int32), 30)   # the same request on its copy
        assert np.array_equal(k0, k1) and np.array_equal(v0, v1)
