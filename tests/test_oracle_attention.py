"""Pins of the oracle's decode attention against brute force, a library
routine, closed forms and invariants.  Also plants typical mistakes in copies
of the oracle and checks that the pins catch each of them.  CPU only."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth


def _rand(seed, n, h_q, h_kv, d, spread=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((h_q, d))
    K = rng.standard_normal((n, h_kv, d)) * spread
    V = rng.standard_normal((n, h_kv, d))
    return q, K, V


SHAPES = [(1, 1, 1, 4), (5, 4, 2, 8), (17, 4, 2, 16), (40, 8, 2, 8), (9, 6, 1, 4),
          (12, 3, 3, 5), (23, 8, 8, 4)]


# -------------------------------------------------------------- pin checks ---
def pin_bruteforce(fn):
    for i, (n, hq, hkv, d) in enumerate(SHAPES):
        q, K, V = _rand(i, n, hq, hkv, d, spread=2.0)
        sc = 1.0 / math.sqrt(d)
        if np.max(np.abs(fn(q, K, V, sc) - oracle.attention_bruteforce(q, K, V, sc))) > 1e-12:
            return False
    return True


def pin_sdpa(fn):
    """torch's scaled_dot_product_attention in float64 on the CPU, with each KV
    head repeated for its G query heads (contiguous groups)."""
    for i, (n, hq, hkv, d) in enumerate(SHAPES):
        q, K, V = _rand(100 + i, n, hq, hkv, d, spread=1.5)
        sc = 0.37
        G = hq // hkv
        tq = torch.from_numpy(q)[:, None, :]                       # [h_q, 1, d]
        tk = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(G, 0)   # [h_q, n, d]
        tv = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(G, 0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.contiguous(), tv.contiguous(), scale=sc)[:, 0, :].numpy()
        if np.max(np.abs(fn(q, K, V, sc) - ref)) > 1e-12:
            return False
    return True


def pin_closed_forms(fn):
    rng = np.random.default_rng(7)
    d = 8
    # identical keys: every weight is 1/n, output is the mean of V
    q = rng.standard_normal((4, d))
    k = rng.standard_normal(d)
    K = np.tile(k, (13, 2, 1))
    V = rng.standard_normal((13, 2, d))
    o = fn(q, K, V, 0.3)
    for h in range(4):
        if np.max(np.abs(o[h] - V[:, h // 2, :].mean(axis=0))) > 1e-12:
            return False
    # one token: output is its value
    K1, V1 = rng.standard_normal((1, 2, d)), rng.standard_normal((1, 2, d))
    o = fn(q, K1, V1, 0.3)
    if np.max(np.abs(o - np.repeat(V1[0], 2, axis=0))) > 1e-15:
        return False
    # one key aligned with q and a huge scale: that token's value wins
    K = rng.standard_normal((9, 1, d)) * 0.01
    qq = rng.standard_normal((1, d))
    K[4, 0] = qq[0] * 10
    V = rng.standard_normal((9, 1, d))
    o = fn(qq, K, V, 50.0)
    if np.max(np.abs(o[0] - V[4, 0])) > 1e-9:
        return False
    # empty cache: zeros
    o = fn(q, np.zeros((0, 2, d)), np.zeros((0, 2, d)), 0.3)
    return o.shape == (4, d) and not np.any(o)


def pin_scale_covariance(fn):
    """Scaling q by c with scale/c leaves the output unchanged; scale 0 gives
    the plain mean of V (checks that the scale enters the exponent)."""
    q, K, V = _rand(3, 11, 4, 2, 8)
    a = fn(q, K, V, 0.5)
    b = fn(q * 4.0, K, V, 0.125)
    m = fn(q, K, V, 0.0)
    ok = np.max(np.abs(a - b)) < 1e-12
    for h in range(4):
        ok &= np.max(np.abs(m[h] - V[:, h // 2, :].mean(0))) < 1e-12
    c = fn(q, K, V, 2.0)
    return bool(ok) and np.max(np.abs(a - c)) > 1e-3


ALL_PINS = [pin_bruteforce, pin_sdpa, pin_closed_forms, pin_scale_covariance]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_oracle_passes_pin(pin):
    assert pin(oracle.attention_fp64)


@pytest.mark.parametrize("part", [1, 3, 16, 100, 512, 10 ** 6])
def test_partitioned_equals_plain(part):
    for i, (n, hq, hkv, d) in enumerate(SHAPES + [(700, 8, 2, 8), (1030, 4, 4, 4)]):
        q, K, V = _rand(200 + i, n, hq, hkv, d, spread=3.0)
        a = oracle.attention_fp64(q, K, V, 0.4)
        b = oracle.partitioned_fp64(q, K, V, 0.4, part)
        assert np.max(np.abs(a - b)) <= 1e-12


def test_batch_and_mha_mqa_cases():
    q, K, V = _rand(5, 30, 8, 8, 4)      # G = 1: every head independent
    o = oracle.attention_fp64(q, K, V, 0.5)
    for h in range(8):
        oh = oracle.attention_fp64(q[h:h + 1], K[:, h:h + 1], V[:, h:h + 1], 0.5)
        assert np.max(np.abs(o[h] - oh[0])) < 1e-15
    q, K, V = _rand(6, 30, 8, 1, 4)      # MQA: one KV head for all
    o = oracle.attention_fp64(q, K, V, 0.5)
    for h in range(8):
        oh = oracle.attention_fp64(q[h:h + 1], K, V, 0.5)
        assert np.max(np.abs(o[h] - oh[0])) < 1e-15
    qs = np.stack([q, q * 2])
    ob = oracle.decode_batch_fp64(qs, [(K, V), (K[:7], V[:7])], 0.5)
    assert np.array_equal(ob[0], o)


def test_shared_prefix_equals_duplicated_pages():
    """Two requests mapping the same prefix pages read the same values as
    requests holding private copies of those pages."""
    rng = np.random.default_rng(11)
    H, D, N = 2, 8, 12
    shared = oracle.RefPool(1, N, H, D, 16, "bf16")
    dup = oracle.RefPool(1, N, H, D, 16, "bf16")
    pre_k = synth.normal_bf16_bits(rng, (32, H, D))
    pre_v = synth.normal_bf16_bits(rng, (32, H, D))
    suf = [(synth.normal_bf16_bits(rng, (5, H, D)), synth.normal_bf16_bits(rng, (5, H, D)))
           for _ in range(2)]
    shared.append(0, pre_k, pre_v, oracle.slot_mapping([0, 1], range(32), 16))
    t_shared = [[0, 1, 2], [0, 1, 3]]
    t_dup = [[4, 5, 6], [7, 8, 9]]
    for i in range(2):
        dup.append(0, pre_k, pre_v, oracle.slot_mapping(t_dup[i][:2], range(32), 16))
        shared.append(0, *suf[i], oracle.slot_mapping(t_shared[i], range(32, 37), 16))
        dup.append(0, *suf[i], oracle.slot_mapping(t_dup[i], range(32, 37), 16))
    q = rng.standard_normal((4, D))
    for i in range(2):
        a = oracle.attention_fp64(q, *shared.gather_f64(0, t_shared[i], 37), 0.35)
        b = oracle.attention_fp64(q, *dup.gather_f64(0, t_dup[i], 37), 0.35)
        assert np.array_equal(a, b)


# ------------------------------------------------------- planted mistakes ----
def _mut_group_mod(q, K, V, scale):          # wrong GQA mapping: h % h_kv
    q, K, V = map(np.asarray, (q, K, V))
    out = np.zeros(q.shape)
    if K.shape[0] == 0:
        return out
    for h in range(q.shape[0]):
        g = h % K.shape[1]
        s = scale * (K[:, g] @ q[h])
        p = np.exp(s - s.max())
        out[h] = (p / p.sum()) @ V[:, g]
    return out


def _mut_no_scale(q, K, V, scale):
    return oracle.attention_fp64(q, K, V, 1.0)


def _mut_swap_kv(q, K, V, scale):            # transposed operand roles
    return oracle.attention_fp64(q, V, K, scale)


def _mut_no_norm(q, K, V, scale):            # dropped normalisation
    q, K, V = map(np.asarray, (q, K, V))
    out = np.zeros(q.shape)
    if K.shape[0] == 0:
        return out
    G = q.shape[0] // K.shape[1]
    for h in range(q.shape[0]):
        s = scale * (K[:, h // G] @ q[h])
        out[h] = np.exp(s - s.max()) @ V[:, h // G]
    return out


def _mut_neg_sign(q, K, V, scale):           # wrong sign in the exponent
    return oracle.attention_fp64(q, K, V, -scale)


def _mut_drop_last(q, K, V, scale):          # off-by-one: last token dropped
    K, V = np.asarray(K), np.asarray(V)
    if K.shape[0] <= 1:
        return oracle.attention_fp64(q, K, V, scale)
    return oracle.attention_fp64(q, K[:-1], V[:-1], scale)


@pytest.mark.parametrize("mut", [_mut_group_mod, _mut_no_scale, _mut_swap_kv, _mut_no_norm,
                                 _mut_neg_sign, _mut_drop_last], ids=lambda f: f.__name__)
def test_pins_catch_planted_mistake(mut):
    assert not all(p(mut) for p in ALL_PINS)
