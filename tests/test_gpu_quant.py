"""8-bit caches (fp8 E4M3 and int8) on the GPU, beyond the N(0,1) inputs of
the other tests ("KV cache and PagedAttention", askaiml §7: the cache stored
as fp8 or int8 with a scale):

* magnitude: K and V scaled by 1e-6 .. 1e6 and q by 1e-5 .. 1e4; every row
  must match the oracle on the dequantised codes to 2e-2 of its largest
  magnitude, the bound the kernel holds at unit scale;
* the codec: kv_append of tiles whose runs hold +-448 (+-127 for int8), so
  the scale is exactly 1, carrying every finite bf16 value in range (and NaN
  for fp8): each code must equal the oracle's encoder byte for byte;
* fp8 end to end: the fp8 workload's batch without outliers against the
  oracle on the inputs before quantisation, the 6e-2 bound;
* decode steps: the last 48 tokens of every request written one per fused
  step, so a tile's scale grows several times and its older codes are
  re-encoded each time; cache bit-exact against the oracle's pool every step,
  and the final decode within the same bounds as above."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import DEV, Case, assert_close, check_indices, from_dev_bits, log, to_dev_bits

pytestmark = pytest.mark.gpu


def _scaled(bits, f):
    """bf16 bits of the values times f (rounded to nearest even)."""
    x = (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64) * f
    return synth.f32_to_bf16_bits(x.astype(np.float32))


def _rowwise_close(got, ref, what, rel=2e-2):
    """|got - ref| <= rel * max|ref| within every (request, head) row."""
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    scale = np.max(np.abs(ref), axis=-1, keepdims=True)
    err = np.abs(got - ref)
    worst = float(np.max(err / np.maximum(scale, np.finfo(np.float64).tiny)))
    log(f"  {what}: worst |err| / max|ref| per row {worst:.3e}")
    assert worst <= rel, f"{what}: {worst:.3e} of the row's magnitude"


class ScaledCase(Case):
    """A Case whose K, V and q bits are scaled before anything is written."""

    def __init__(self, dtype, H, D, h_q, lens, fk, fv, fq, seed):
        self._f = (fk, fv, fq)
        super().__init__(dtype, H, D, h_q, lens, seed=seed, mirror=True)

    def append_host(self, k, v, slots):
        fk, fv, fq = self._f
        self.k, self.v = _scaled(k, fk), _scaled(v, fv)
        self.q = _scaled(self.q, fq)
        super().append_host(self.k, self.v, slots)


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
@pytest.mark.parametrize("fkv,fq", [(1e-6, 1.0), (1e-4, 1.0), (1.0, 1.0), (1e4, 1.0), (1e6, 1.0),
                                    (1.0, 1e-5), (1.0, 1e4), (1e-6, 1e4), (1e6, 1e-5)])
def test_magnitudes(gpu_lib, dtype, fkv, fq):
    lens = [33, 700, 1500, 17, 260]
    c = ScaledCase(dtype, 2, 128, 8, lens, fkv, fkv, fq, seed=31)
    ref = c.oracle()
    for part in (0, 64):   # many pieces per request (reduce kernel), then few (merged in the decode)
        got = c.decode(partition_tokens=part)
        for b in range(len(lens)):
            _rowwise_close(got[b], ref[b], f"{dtype} K,V x{fkv:g} q x{fq:g} part {part} ctx {lens[b]}")


def _codec_tiles(values, vmax, nan=False):
    """Token rows [T, 1, 128] covering `values`, 16 tokens per tile; every
    tile holds +vmax and -vmax (so its scale is exactly 1) and, for fp8, NaN."""
    per_tile = 16 * 128 - 2 - (2 if nan else 0)
    tiles = []
    for i in range(0, len(values), per_tile):
        chunk = np.asarray(values[i:i + per_tile], np.uint16)
        fill = np.full(16 * 128, synth.f32_to_bf16_bits(np.float32(0.0)), np.uint16)
        extra = [vmax, -vmax] + ([np.nan, -np.nan] if nan else [])
        head = synth.f32_to_bf16_bits(np.array(extra, np.float32))
        fill[:len(head)] = head
        fill[len(head):len(head) + len(chunk)] = chunk
        tiles.append(fill.reshape(16, 1, 128))
    return np.concatenate(tiles)


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_codec_every_bf16_value(gpu_lib, dtype):
    vmax = 448.0 if dtype == "fp8" else 127.0
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = (bits.astype(np.uint32) << 16).view(np.float32)
    keep = np.isfinite(vals) & (np.abs(vals) <= vmax)
    values = bits[keep]
    rows = _codec_tiles(values, vmax, nan=(dtype == "fp8"))
    T = rows.shape[0]
    N = T // 16
    c = Case(dtype, 1, 128, 1, [0], num_blocks=N, order=np.arange(N), seed=0, mirror=False)
    slots = np.arange(T, dtype=np.int32)
    d_slots = torch.from_numpy(slots).to(DEV)
    c.pool.append(0, to_dev_bits(rows, "bf16"), to_dev_bits(rows[::-1].copy(), "bf16"), d_slots)
    torch.cuda.synchronize()
    ks, vs = c.pool.k_scale.cpu().numpy()[0, :, 0], c.pool.v_scale.cpu().numpy()[0, :, 0]
    assert np.all(ks == 1.0) and np.all(vs == 1.0)
    x = (rows.astype(np.uint32) << 16).view(np.float32)                  # [T, 1, 128]
    enc = oracle.e4m3_encode if dtype == "fp8" else (lambda y: oracle.int8_encode(y).view(np.uint8))
    want_k = enc(x)
    want_v = enc(x[::-1])
    kc = c.pool.k_cache.cpu().numpy().view(np.uint8)[0]                   # [N, 1, 16, 128]
    vc = c.pool.v_cache.cpu().numpy().view(np.uint8)[0]                   # [N, 1, 128, 16]
    got_k = kc.reshape(T, 1, 128)
    got_v = vc.transpose(0, 1, 3, 2).reshape(T, 1, 128)
    bad = int(np.sum(got_k != want_k)) + int(np.sum(got_v != want_v))
    log(f"{dtype}: {values.size} finite bf16 values in [-{vmax:g}, {vmax:g}] over {N} tiles, "
        f"{bad} codes differ")
    assert bad == 0
    # the oracle's own pool gives the same bytes (scale rule and layout)
    ref = oracle.RefPool(1, N, 1, 128, 16, dtype)
    ref.append(0, rows, rows[::-1].copy(), slots)
    assert np.array_equal(kc, ref.K[0].view(np.uint8)) and np.array_equal(vc, ref.V[0].view(np.uint8))


def test_fp8_end_to_end_without_outliers(gpu_lib):
    """The fp8 workload's batch (128 requests of 1k-8k tokens) with N(0,1)
    values and no outliers: the decode against the fp64 oracle on the bf16
    inputs before quantisation, max |err| <= 6e-2, both splits."""
    w = synth.WORKLOADS["fp8"]
    rng = synth.streams(5)
    lens = synth.uniform_contexts(rng["contexts"], w["batch"], *w["ctx_range"])
    N = int(sum(oracle.blocks_for(int(n), 16) for n in lens))
    c = Case("fp8", w["h_kv"], w["head_dim"], w["h_q"], lens, num_blocks=N,
             order=synth.permutation(rng["free_order"], N), seed=55, device_inputs=True,
             max_blocks=512, outlier_p=0.0, mirror=False)
    got = {part: c.decode(partition_tokens=part) for part in (0, w["partition_tokens"])}
    q = c.q_f64()
    scale = 1.0 / math.sqrt(w["head_dim"])
    worst = 0.0
    for b in [int(x) for x in rng["q"].choice(len(lens), 6, replace=False)] + [int(np.argmax(lens))]:
        kraw, vraw = c.seq_raw(b)
        ref0 = oracle.attention_fp64(q[b], oracle.bf16_bits_to_f64(kraw), oracle.bf16_bits_to_f64(vraw), scale)
        for part, o in got.items():
            err = float(np.max(np.abs(o[b] - ref0)))
            worst = max(worst, err)
            log(f"  request {b} (ctx {int(lens[b])}) partition {part}: max|kernel - oracle(inputs)| {err:.3e}")
            assert np.all(np.isfinite(o[b])) and err <= 6e-2
    log(f"fp8 end to end, no outliers: worst {worst:.3e} (bound 6e-2)")


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_end_to_end_after_decode_steps(gpu_lib, dtype):
    """Requests of the fp8 workload's shape (h_q 32, h_kv 8, d 128; 1k-2k
    tokens), N(0,1) values without outliers, whose last 48 tokens arrive one
    per fused decode step.  Each single-token append may grow its tile's scale
    and re-encode the tile's older codes from their decoded values, so those
    codes are rounded more than once.  Every step the cache must equal the
    oracle pool's bit for bit (checked inside decode_append_step); after the
    last step the output must match the oracle on the stored codes (the
    dtype's tolerance) and stay within 6e-2 of the oracle on the inputs before
    quantisation."""
    w = synth.WORKLOADS[dtype]
    rng = synth.streams(71)
    B, steps = 12, 48
    lens = synth.uniform_contexts(rng["contexts"], B, 1024, 2048)
    N = int(sum(oracle.blocks_for(int(n) + steps, 16) for n in lens))
    c = Case(dtype, w["h_kv"], w["head_dim"], w["h_q"], lens, num_blocks=N,
             order=synth.permutation(rng["free_order"], N), seed=72, max_blocks=oracle.blocks_for(2048 + steps, 16),
             mirror=True)
    o = None
    for i in range(steps):
        o = c.decode_append_step(seed=1000 + i)
    ref_codes = c.oracle(dequant=True)
    ref_inputs = c.oracle(dequant=False)
    worst = 0.0
    for b in range(B):
        assert_close(o[b], ref_codes[b], c.tol_key, f"request {b} against the stored codes")
        err = float(np.max(np.abs(o[b] - ref_inputs[b])))
        worst = max(worst, err)
        assert np.all(np.isfinite(o[b])) and err <= 6e-2, f"request {b}: {err:.3e} against the inputs"
    log(f"{dtype} after {steps} decode steps: worst |kernel - oracle(inputs)| {worst:.3e} (bound 6e-2)")
