"""Pins of the sliding-window / attention-sink oracle: special cases with a
known answer, brute force over explicit position lists, invariance to the
excluded positions, the memory formula's printed example, and a brute-force
definition of a dead page (no later request length reads it).  Planted
off-by-one mistakes must fail them."""

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
