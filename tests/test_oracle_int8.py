"""Pins of the INT8 cache oracle: round-half-even ties, the symmetric clamp,
exact round trips of every code, the half-step error bound of the scale rule
(including re-encoding when a tile's scale grows), the amax element hitting
+-127, and the byte-level pool model.  Planted mistakes (truncation, an
asymmetric clamp) must fail them."""

import numpy as np
import pytest

import oracle
from oracle import int8 as Q

# x * (1/s) is formed in fp32 before rounding: |code| <= 127, so the product
# may be off by 127 * 2^-23 of a step beyond the half step
HALF = 0.5 + 127 * 2.0 ** -23


def test_ties_round_to_even_and_clamp_is_symmetric():
    y = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 126.5, 127.49, 127.5, 300.0, -127.5, -300.0],
                 np.float32)
    want = [0, 2, 2, 4, 0, -2, -2, 126, 127, 127, 127, -127, -127]
    assert Q.int8_encode(y).tolist() == want


def test_every_code_round_trips():
    c = np.arange(-127, 128, dtype=np.int8)
    assert np.array_equal(Q.int8_encode(Q.int8_decode(c).astype(np.float32)), c)
    assert Q.int8_decode(c).tolist() == list(range(-127, 128))


def test_run_error_bound_and_amax_code():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((12, 64)).astype(np.float32) * 3
    codes, _, s = Q.quantize_run_int8(x, np.zeros((16, 64), np.int8), 0.0, 0)
    assert s == np.float32(np.abs(x).max() / np.float32(127))
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert abs(int(codes[i])) == 127
    err = np.abs(codes.astype(np.float64) * float(s) - x)
    assert err.max() <= float(s) * HALF


def test_scale_growth_reencodes_below_the_run():
    rng = np.random.default_rng(2)
    first = rng.standard_normal((5, 32)).astype(np.float32)
    tile = np.zeros((16, 32), np.int8)
    c1, tile, s0 = Q.quantize_run_int8(first, tile, 0.0, 0)
    tile[:5] = c1
    big = (4 * rng.standard_normal((3, 32))).astype(np.float32)
    c2, tile2, s1 = Q.quantize_run_int8(big, tile, s0, 5)
    assert s1 > s0
    old = tile[:5].astype(np.float64) * float(s0)
    # the re-encoded codes stay within half a new step of the old values
    assert np.abs(tile2[:5].astype(np.float64) * float(s1) - old).max() <= float(s1) * HALF
    # a run that does not grow the scale leaves the old codes alone
    small = (0.01 * rng.standard_normal((2, 32))).astype(np.float32)
    _, tile3, s2 = Q.quantize_run_int8(small, tile2, s1, 8)
    assert s2 == s1 and np.array_equal(tile3, tile2)


def test_zero_run_gives_zero_codes():
    codes, tile, s = Q.quantize_run_int8(np.zeros((3, 8), np.float32), np.zeros((16, 8), np.int8), 0.0, 0)
    assert s == 0 and not codes.any()


def test_pool_model_int8():
    rng = np.random.default_rng(3)
    H, D = 2, 64
    ref = oracle.RefPool(1, 4, H, D, 16, "int8")
    import synth
    kb = synth.normal_bf16_bits(rng, (20, H, D), 0.05, 8.0)
    vb = synth.normal_bf16_bits(rng, (20, H, D))
    slots = np.concatenate([np.arange(16) + 32, np.arange(4) + 16])   # block 2, then block 1
    ref.append(0, kb, vb, slots)
    K, V = ref.gather_f64(0, [2, 1], 20)
    K0, V0 = oracle.bf16_bits_to_f64(kb), oracle.bf16_bits_to_f64(vb)
    for blk, rows in ((2, slice(0, 16)), (1, slice(16, 20))):
        for g in range(H):
            s = float(ref.Ks[0, blk, g])
            assert np.abs(K[rows, g] - K0[rows, g]).max() <= s * HALF
            sv = float(ref.Vs[0, blk, g])
            assert np.abs(V[rows, g] - V0[rows, g]).max() <= sv * HALF


def test_planted_mistakes_fail():
    orig = Q.int8_encode
    try:
        Q.int8_encode = lambda y: np.clip(np.trunc(np.asarray(y, np.float32)), -127, 127).astype(np.int8)
        with pytest.raises(AssertionError):
            test_ties_round_to_even_and_clamp_is_symmetric()
        Q.int8_encode = lambda y: np.clip(np.rint(np.asarray(y, np.float32)), -128, 127).astype(np.int8)
        with pytest.raises(AssertionError):
            test_ties_round_to_even_and_clamp_is_symmetric()
    finally:
        Q.int8_encode = orig
