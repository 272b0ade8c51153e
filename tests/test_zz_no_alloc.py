"""paged_attention_decode_append_noalloc (the fused decode step with the
library's fixed scratch in place of a caller workspace) against
paged_attention_decode_append with a caller workspace: two twin pools built
from the same seeds, one fused step on each, twice in a row (the second
batch smaller, with a different split and merge path); outputs and the
caches the steps wrote must agree bit for bit, and each output matches the
fp64 oracle."""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_271_amd as pk
from gpu_cases import DEV, Case, assert_close, check_indices, check_slots, from_dev_bits, log, to_dev_bits

pytestmark = pytest.mark.gpu


def _step(c, noalloc, seed):
    """One fused step on Case c (every request appends one token)."""
    B = len(c.lens_list)
    slots = c.pool.batch_reserve(c.table, c.lens, np.ones(B, np.int32))
    check_slots(slots, c.N)
    c.sync_tables()
    max_ctx = int(c.lens.max())
    check_indices(c.table, c.lens, c.N, max_ctx)
    rng = np.random.default_rng(seed)
    import synth
    k = synth.normal_bf16_bits(rng, (B, c.H, c.D))
    v = synth.normal_bf16_bits(rng, (B, c.H, c.D))
    q = to_dev_bits(c.q, "bf16")
    out = torch.full(tuple(q.shape), float("nan"), dtype=q.dtype, device=DEV)
    args = (c.pool.handle, c.pool.desc, 0, out, q, to_dev_bits(k, "bf16"), to_dev_bits(v, "bf16"),
            torch.from_numpy(slots).to(DEV), c.d_table, c.d_lens, max_ctx, 1.0 / math.sqrt(c.D))
    if noalloc:
        pk.paged_attention_decode_append_noalloc(*args)
    else:
        ws = c.pool.new_workspace(B, c.h_q, max_ctx)
        pk.paged_attention_decode_append(*args, 0, ws)
    torch.cuda.synchronize()
    c._seqs = [(np.concatenate([kb, k[b:b + 1]]), np.concatenate([vb, v[b:b + 1]]))
               for b, (kb, vb) in enumerate(c.seq_raw(b) for b in range(B))]
    c.lens_list = [n + 1 for n in c.lens_list]
    return from_dev_bits(out)


@pytest.mark.parametrize("lens_a,lens_b", [
    (list(np.random.default_rng(91).integers(300, 2500, 64)), [17, 400, 1, 900, 33, 2000, 64, 5]),
])
def test_noalloc_matches_workspace_call(gpu_lib, lens_a, lens_b):
    for lens, seed in ((lens_a, 92), (lens_b, 93)):       # two calls in a row, the second smaller
        N = sum(oracle.blocks_for(int(n), 16) for n in lens) + len(lens)   # room for the step's tokens
        MB = max(oracle.blocks_for(int(n) + 1, 16) for n in lens)
        twins = [Case("bf16", 8, 128, 32, lens, num_blocks=N, max_blocks=MB, seed=seed) for _ in range(2)]
        outs = [_step(c, noalloc=(i == 1), seed=seed + 100) for i, c in enumerate(twins)]
        a, b = outs
        assert np.all(np.isfinite(oracle.bf16_bits_to_f64(b)))
        assert np.array_equal(a, b), "no-allocation call differs from the workspace call"
        for name in ("k_cache", "v_cache"):
            ta, tb = getattr(twins[0].pool, name), getattr(twins[1].pool, name)
            assert torch.equal(ta.view(torch.int16), tb.view(torch.int16)), f"{name} differs"
        got = oracle.bf16_bits_to_f64(b)
        c = twins[1]
        sample = sorted({0, len(lens) - 1, int(np.argmax(lens))})
        ref = c.oracle(batch=sample)
        for r in sample:
            assert_close(got[r], ref[r], "bf16", f"no-allocation step, B {len(lens)}, request {r} ({c.lens_list[r]} tokens)")
        log(f"B={len(lens)}: no-allocation step equals the workspace step bit for bit")


def test_noalloc_rejects_oversized_batch(gpu_lib):
    pool = pk.Pool(1, 64, 8, 128, "bf16", DEV)
    B, h_q = 8192, 8 * 16                     # 16 query heads per kv head: about 51 MB of states
    assert pool.workspace_bytes(B, h_q, 16) > 24 << 20
    q = torch.zeros((B, h_q, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((B, 8, 128), dtype=torch.bfloat16, device=DEV)
    slots = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    table = torch.zeros((B, 1), dtype=torch.int32, device=DEV)
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    with pytest.raises(pk.KVError) as e:
        pk.paged_attention_decode_append_noalloc(pool.handle, pool.desc, 0, torch.empty_like(q), q, kv, kv, slots,
                                                 table, lens, 16, 0.1)
    assert e.value.name == "KV_E_WORKSPACE" and "scratch" in str(e.value)
