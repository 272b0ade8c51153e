"""Symmetric INT8 codec and the per-tile scale rule of the int8 cache (oracle;
test infrastructure).

Follows "KV cache and PagedAttention" (askaiml.pages.dev), §7 "KV cache
quantisation": INT8 KV sits next to fp8 E4M3 as a cheaper cache format with
similar quality and broader hardware support; the "KV Cache" glossary
(inferensys.com) lists FP8 or INT8 cache quantization as the common way to
compress the cache.

Readings taken where the pages give only the name:
* Symmetric codes with one fp32 scale per (layer, block, kv-head), separately
  for K and V, and the same tile-run rule as the fp8 cache with 127 in place
  of 448: for the tokens of one append call that land in one tile, s1 =
  max(s0, max|x| / 127) (s0 = 0 for a run starting at offset 0, else the
  stored scale); codes already in the tile below the run are re-encoded from
  code * s0 when s1 != s0.
* code = clamp(round_half_even(x * (1 / s1)), -127, 127), the product and the
  reciprocal in fp32 (the reciprocal correctly rounded); -128 is never
  produced, so the code range is symmetric.  s1 == 0 gives code 0.  Inputs are
  finite.
* The stored value is code * scale.
"""

import numpy as np

INT8_MAX = 127


def int8_encode(y):
    """float32 values (already divided by the scale) -> int8 codes."""
    r = np.rint(np.asarray(y, dtype=np.float32))      # round half to even
    return np.clip(r, -INT8_MAX, INT8_MAX).astype(np.int8)


def int8_decode(codes):
    return np.asarray(codes, dtype=np.int8).astype(np.float64)


def quantize_run_int8(x_run, tile_codes, s0, first_offset):
    """The tile rule for one run of one tile (arguments and results as
    fp8.quantize_run, with int8 codes)."""
    x_run = np.asarray(x_run, dtype=np.float32)
    s0 = np.float32(0.0) if first_offset == 0 else np.float32(s0)
    amax = np.float32(np.max(np.abs(x_run))) if x_run.size else np.float32(0.0)
    s1 = np.float32(max(s0, np.float32(amax / np.float32(INT8_MAX))))
    tile = np.array(tile_codes, dtype=np.int8, copy=True)
    if s1 == np.float32(0.0):
        return np.zeros(x_run.shape, dtype=np.int8), tile, s1
    inv = np.float32(np.float32(1.0) / s1)
    if s1 != s0 and first_offset > 0:
        old = tile[:first_offset].astype(np.float32) * s0
        tile[:first_offset] = int8_encode((old * inv).astype(np.float32))
    codes = int8_encode((x_run * inv).astype(np.float32))
    return codes, tile, s1
