"""FP8 E4M3 codec and the per-tile scale rule of the fp8 cache (oracle; test
infrastructure).

The pages name the format only ("fp8 KV (E4M3)", halving the bytes:
"KV cache and PagedAttention" (askaiml.pages.dev), §7 "KV cache quantisation";
FP8/INT8 compression in the "KV Cache" glossary (inferensys.com), trade-offs).
The format itself is the OCP 8-bit floating point E4M3 encoding (OFP8
specification 1.0): 1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
exponent field 0 holds subnormals m * 2^-9; the single all-ones pattern
S.1111.111 is NaN; there are no infinities; the largest finite magnitude is
S.1111.110 = 1.75 * 2^8 = 448.

Encoding reading (the pages give none): round to nearest, ties to the code with
an even mantissa, magnitudes at or above 448 (infinity included) saturate to
448, NaN maps to S.1111.111, and the sign is kept (so tiny negative values give
the negative-zero code 0x80).

Scale rule (the pages give none; one fp32 scale per (layer, block, kv-head) for
K and another for V).  A "run" is the set of tokens of one append call that land
in the same (block, kv-head) tile; they are consecutive tokens of the call.

* s0 is the tile's stored scale, except that a run whose first token lands at
  offset 0 starts a fresh tile: then s0 = 0 and nothing is re-encoded.
* amax = max |x| over the run (fp32), s1 = max(s0, amax / 448) in fp32.  A NaN
  in the run does not set the scale: both maxima skip NaN operands, as IEEE
  maxNum does (the NaN itself is then encoded as the NaN code).
* If s1 != s0, every slot of the tile below the run's first offset is
  re-encoded: value = decode(code) * s0 (fp32), code = encode(value * (1/s1)).
* New codes: encode(x * (1/s1)) with the fp32 reciprocal correctly rounded;
  if s1 == 0 every code is 0.
* Dequantised value: decode(code) * s.

All fp32 steps are single IEEE operations on numpy float32 scalars/arrays, each
rounded to nearest-even, in the order written above.
"""

import numpy as np

E4M3_MAX = 448.0
_NAN_CODE = 0x7F


def _decode_one(code):
    s = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9          # subnormal: (m / 8) * 2^(1 - 7)
    return s * (1.0 + m / 8.0) * 2.0 ** (e - 7)


_TABLE = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)
# non-negative finite codes 0x00..0x7E in increasing order of value
_POS_VALUES = _TABLE[:0x7F].copy()


def e4m3_value_table():
    """All 256 codes decoded to float64 (NaN for the two NaN codes)."""
    return _TABLE.copy()


def e4m3_decode(codes):
    """uint8 codes -> float64 values."""
    return _TABLE[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x):
    """float32 (or float64) values -> uint8 E4M3 codes, RNE, saturating."""
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    sign = np.signbit(flat)
    a = np.abs(flat)
    nan = np.isnan(flat)
    sat = ~nan & (a >= E4M3_MAX)
    mid = ~nan & ~sat
    am = a[mid]
    # index of the first table value >= a; candidates are idx-1 and idx
    hi = np.searchsorted(_POS_VALUES, am, side="left")
    hi = np.clip(hi, 0, len(_POS_VALUES) - 1)
    lo = np.clip(hi - 1, 0, None)
    d_hi = _POS_VALUES[hi] - am
    d_lo = am - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(_POS_VALUES[hi] == am, hi, code)   # exact hit
    out[mid] = code.astype(np.uint8)
    out[sat] = 0x7E
    out[nan] = _NAN_CODE
    out |= (sign.astype(np.uint8) << 7)
    return out.reshape(x.shape)


def quantize_run(x_run, tile_codes, s0, first_offset):
    """Apply the tile scale rule for one run of one tile.

    x_run:       float32 [n_run, ...] new values (bf16 inputs already widened
                 to float32 exactly).
    tile_codes:  uint8 array of the tile's current codes indexed as
                 [offset, ...]; slots below first_offset are re-encoded in a
                 copy if the scale grows.
    s0:          stored fp32 scale of the tile.
    first_offset: offset in the tile of the run's first token.

    Returns (new_codes_for_run uint8 [n_run, ...], updated_tile_codes, s1).
    """
    x_run = np.asarray(x_run, dtype=np.float32)
    s0 = np.float32(0.0) if first_offset == 0 else np.float32(s0)
    # maxNum: NaN operands are skipped (the result is NaN only if all are NaN)
    amax = np.float32(np.fmax.reduce(np.abs(x_run).ravel())) if x_run.size else np.float32(0.0)
    s1 = np.float32(np.fmax(s0, np.float32(amax / np.float32(E4M3_MAX))))
    tile = np.array(tile_codes, dtype=np.uint8, copy=True)
    if s1 == np.float32(0.0):
        return np.zeros(x_run.shape, dtype=np.uint8), tile, s1
    inv = np.float32(np.float32(1.0) / s1)
    if s1 != s0 and first_offset > 0:
        old = e4m3_decode(tile[:first_offset]).astype(np.float32) * s0
        tile[:first_offset] = e4m3_encode((old * inv).astype(np.float32))
    codes = e4m3_encode((x_run * inv).astype(np.float32))
    return codes, tile, s1
