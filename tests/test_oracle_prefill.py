"""Pins of the causal prefill oracle: one query is the decode step, scalar
brute force of the causal sum, the last query seeing everything, keys after
a query never mattering to it, the FLOP count's closed form, and a planted
off-by-one in the causal bound."""

import math

import numpy as np
import pytest

import oracle
from oracle import prefill as PF


def data(rng, n, P, h_q=4, h_kv=2, d=8):
    return (rng.standard_normal((P, h_q, d)), rng.standard_normal((n, h_kv, d)),
            rng.standard_normal((n, h_kv, d)))


def test_one_query_is_the_decode_step():
    rng = np.random.default_rng(1)
    q, K, V = data(rng, 23, 1)
    assert np.array_equal(PF.prefill_attention_fp64(q, K, V, 0.3)[0], oracle.attention_fp64(q[0], K, V, 0.3))


def test_causal_bruteforce():
    rng = np.random.default_rng(2)
    n, P = 9, 5
    q, K, V = data(rng, n, P)
    got = PF.prefill_attention_fp64(q, K, V, 0.5)
    G = 2
    for i in range(P):
        pos = n - P + i
        for h in range(4):
            g = h // G
            s = [0.5 * math.fsum(q[i, h, k] * K[t, g, k] for k in range(8)) for t in range(pos + 1)]
            m = max(s)
            e = [math.exp(x - m) for x in s]
            den = math.fsum(e)
            for k in range(8):
                want = math.fsum(e[t] * V[t, g, k] for t in range(pos + 1)) / den
                assert abs(got[i, h, k] - want) < 1e-12


def test_last_query_reads_everything_and_future_keys_do_not_matter():
    rng = np.random.default_rng(3)
    n, P = 40, 40
    q, K, V = data(rng, n, P)
    a = PF.prefill_attention_fp64(q, K, V, 0.3)
    assert np.allclose(a[-1], oracle.attention_fp64(q[-1], K, V, 0.3), atol=1e-14)
    K2, V2 = K.copy(), V.copy()
    K2[20:] = 100 * rng.standard_normal(K2[20:].shape)
    V2[20:] = np.nan
    b = PF.prefill_attention_fp64(q, K2, V2, 0.3)
    assert np.array_equal(a[:20], b[:20])


def test_flop_count_closed_form():
    # P new tokens after C cached: keys read = C*P + P(P+1)/2
    for C, P in ((0, 1), (0, 2048), (30, 10), (500, 129)):
        assert PF.prefill_flops([C + P], [P], 32, 128) == (C * P + P * (P + 1) // 2) * 32 * 4 * 128


def test_planted_off_by_one_fails():
    orig = PF.prefill_attention_fp64

    def wrong(q, K, V, scale):
        q = np.asarray(q, np.float64)
        P, n = q.shape[0], len(K)
        out = np.zeros(q.shape)
        for i in range(P):
            pos = n - P + i
            out[i] = oracle.attention_fp64(q[i], K[:pos], V[:pos], scale)   # misses itself
        return out
    PF.prefill_attention_fp64 = wrong
    try:
        with pytest.raises(AssertionError):
            test_one_query_is_the_decode_step()
    finally:
        PF.prefill_attention_fp64 = orig
