"""Pins of the oracle's E4M3 codec and per-tile scale rule.  CPU only."""

import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _landmarks():
    with open(os.path.join(GOLDEN, "ocp_e4m3_landmarks.json")) as f:
        return json.load(f)


def test_landmarks_from_spec():
    g = _landmarks()
    t = oracle.e4m3_value_table()
    for lm in g["landmarks"]:
        c = int(lm["code"], 16)
        assert t[c] == lm["value"] and np.signbit(t[c]) == np.signbit(lm["value"]), lm
        assert oracle.e4m3_encode(np.float32(lm["value"])) == c
    for c in g["nan_codes"]:
        assert np.isnan(t[int(c, 16)])
    assert np.isnan(t).sum() == 2
    assert oracle.E4M3_MAX == 448.0


def test_table_monotone_and_symmetric():
    t = oracle.e4m3_value_table()
    pos = t[:0x7F]
    assert np.all(np.diff(pos) > 0)
    assert np.array_equal(t[0x80:0xFF], -pos)


def test_roundtrip_every_finite_code():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    assert np.array_equal(oracle.e4m3_encode(oracle.e4m3_decode(codes).astype(np.float32)), codes)


def test_midpoints_tie_to_even_and_neighbours():
    pos = oracle.e4m3_value_table()[:0x7F]
    for c in range(0x7E):
        mid = np.float32((pos[c] + pos[c + 1]) / 2)        # exact in fp32
        assert float(mid) == (pos[c] + pos[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert oracle.e4m3_encode(mid) == even
        assert oracle.e4m3_encode(-mid) == even | 0x80
        below = np.nextafter(mid, np.float32(0))
        above = np.nextafter(mid, np.float32(1000))
        assert oracle.e4m3_encode(below) == c
        assert oracle.e4m3_encode(above) == c + 1


def test_saturation_nan_and_signed_zero():
    x = np.array([448, 449, 464, 1e6, np.inf, -500, -np.inf, np.nan, -1e-30, 1e-30],
                 np.float32)
    assert oracle.e4m3_encode(x).tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE,
                                              0x7F, 0x80, 0x00]


def test_agrees_with_torch_float8_in_range():
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even) as an
    independent implementation, inside the finite range."""
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * np.float32(30),
        rng.standard_normal(50000).astype(np.float32) * np.float32(0.01),
        (rng.random(50000) * 896 - 448).astype(np.float32)])
    x = x[np.abs(x) < 448]
    ours = oracle.e4m3_encode(x)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_fresh_tile_scale_and_error_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((16, 128)) * 3).astype(np.float32)
    x[3, 7] = np.float32(-25.0)
    codes, tile, s = oracle.quantize_run(x, np.zeros((16, 128), np.uint8), 0.0, 0)
    assert s == np.float32(np.float32(25.0) / np.float32(448.0))
    assert codes[3, 7] == 0xFE                    # the extreme lands on -448
    back = oracle.e4m3_decode(codes) * np.float64(s)
    err = np.abs(back - x)
    # half an E4M3 step: 2^-4 relative in the normal range, 2^-10 * s below it
    assert np.all(err <= np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * float(s)) * (1 + 1e-6))


def test_scale_grows_and_reencodes_earlier_slots():
    x1 = np.full((3, 4), 1.0, np.float32)
    codes1, tile, s1 = oracle.quantize_run(x1, np.zeros((16, 4), np.uint8), 0.0, 0)
    tile[0:3] = codes1
    assert s1 == np.float32(1.0) / np.float32(448.0) and np.all(codes1 == 0x7E)
    x2 = np.full((1, 4), 4.0, np.float32)
    codes2, tile2, s2 = oracle.quantize_run(x2, tile, s1, 3)
    assert s2 == np.float32(4.0) / np.float32(448.0)
    assert np.all(codes2 == 0x7E)
    # earlier values 1.0 now encode 112 = 1.75 * 2^6
    assert np.all(oracle.e4m3_decode(tile2[:3]) == 112.0)
    assert np.array_equal(tile2[3:], tile[3:])
    # a smaller value keeps the scale and leaves earlier codes alone
    codes3, tile3, s3 = oracle.quantize_run(np.full((1, 4), 0.5, np.float32), tile2, s2, 4)
    assert s3 == s2 and np.array_equal(tile3, tile2)
    # a run starting at offset 0 ignores the stale scale
    _, _, s4 = oracle.quantize_run(np.full((1, 4), 0.5, np.float32), tile2, s2, 0)
    assert s4 == np.float32(0.5) / np.float32(448.0)


def test_zero_run_gives_zero_codes():
    codes, _, s = oracle.quantize_run(np.zeros((2, 8), np.float32), np.zeros((16, 8), np.uint8), 0.0, 0)
    assert s == 0 and not codes.any()


def test_pool_fp8_append_runs():
    """Appending token by token and appending in one call reach the same
    scales when the first token holds the tile maximum."""
    H, D = 2, 8
    rng = np.random.default_rng(3)
    x = rng.standard_normal((16, H, D)).astype(np.float32)
    x[0] *= 10
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)     # truncation: exact bf16 inputs
    a = oracle.RefPool(1, 2, H, D, 16, "fp8")
    b = oracle.RefPool(1, 2, H, D, 16, "fp8")
    a.append(0, bits, bits, np.arange(16) + 16)
    for t in range(16):
        b.append(0, bits[t:t + 1], bits[t:t + 1], [16 + t])
    assert np.array_equal(a.Ks, b.Ks) and np.array_equal(a.K, b.K)
    assert np.array_equal(a.Vs, b.Vs) and np.array_equal(a.V, b.V)
    kd, vd = a.gather_f64(0, [1], 16)
    xin = ((bits.astype(np.uint32) << 16).view(np.float32)).astype(np.float64)
    assert np.max(np.abs(kd - xin)) <= np.max(np.abs(xin)) / 448 * 16
    assert np.array_equal(kd, vd)


def test_nan_in_a_run_does_not_set_the_scale():
    """A NaN among a run's values: the scale and the other codes are those of
    the run without it (maxNum skips NaN), and the NaN takes the NaN code
    with its sign."""
    from oracle import fp8
    rng = np.random.default_rng(7)
    x = rng.standard_normal((5, 2, 8)).astype(np.float32)
    x[1, 0, 3] = np.nan
    x[3, 1, 0] = -np.nan
    tile = np.zeros((16, 2, 8), np.uint8)
    codes, _, s1 = fp8.quantize_run(x, tile, np.float32(0), 0)
    finite = np.isfinite(x)
    assert s1 == np.float32(np.max(np.abs(x[finite])) / np.float32(448.0))
    clean = np.where(finite, x, np.float32(0))
    codes_clean, _, s_clean = fp8.quantize_run(clean, tile, np.float32(0), 0)
    assert s_clean == s1
    assert np.array_equal(codes[finite], codes_clean[finite])
    assert codes[1, 0, 3] == 0x7F and codes[3, 1, 0] == 0xFF
    # the largest magnitude maps to +-448 (code 0x7E / 0xFE) at this scale
    k = np.unravel_index(np.argmax(np.where(finite, np.abs(x), 0)), x.shape)
    assert codes[k] & 0x7F == 0x7E
