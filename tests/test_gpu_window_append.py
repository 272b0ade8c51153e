"""GPU parity of paged_attention_decode_window_append (one sliding-window
decode step with the step's append) against the fp64 oracle: the output over
the sinks and the window of the grown contexts, the cache bytes the call
leaves, requests that append nothing, pages released by kv_window_release
and then poisoned (bf16: a read of one would show as NaN), both work splits,
and agreement with kv_append followed by paged_attention_decode_window."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import Case, DEV, NAN_BITS, assert_close, log, to_dev_bits

pytestmark = pytest.mark.gpu

# final context lengths of the first step: a lone new token, block edges, a
# new token opening a fresh page, long requests that span several pieces
FINAL = [1, 2, 15, 16, 17, 33, 100, 333, 1000]
SKIP = (3, 6)   # these requests append nothing and decode what they hold


def _case(dtype, H, h_q, seed, sink, win, poison):
    appends = np.array([i not in SKIP for i in range(len(FINAL))])
    prefill = [n - int(a) for n, a in zip(FINAL, appends)]
    N = sum(oracle.blocks_for(n + 2, 16) for n in FINAL) + 3
    mb = oracle.blocks_for(max(FINAL) + 2, 16)
    c = Case(dtype, H, 128, h_q, prefill, num_blocks=N, order=np.random.default_rng(seed).permutation(N),
             seed=seed, max_blocks=mb, poison=poison and dtype == "bf16")
    before = c.table.copy()
    n_rel = c.pool.window_release(c.table, c.lens, sink, win)
    assert n_rel == sum(len(oracle.dead_pages(n, sink, win)) for n in prefill)
    pages = sorted({int(x) for x in before[before != c.table]})
    if poison and dtype == "bf16" and pages:
        idx = torch.tensor(pages, dtype=torch.int64, device=DEV)
        c.pool.k_cache.view(torch.int16)[0, idx] = NAN_BITS["bf16"]
        c.pool.v_cache.view(torch.int16)[0, idx] = NAN_BITS["bf16"]
    c.sync_tables()
    return c, appends


def _check(c, got, sink, win, what):
    q = c.q_f64()
    scale = 1.0 / math.sqrt(c.D)
    assert np.all(np.isfinite(got)), what
    for b, n in enumerate(c.lens_list):
        if n == 0:
            continue
        K, V = c.seq_f64(b)
        ref = oracle.attention_window_fp64(q[b], K, V, scale, sink, win)
        assert_close(got[b], ref, c.tol_key, f"{what} ctx {n}")


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("sink,win", [(0, 1), (4, 16), (4, 100), (17, 33), (0, 5000), (40, 7), (16, 16)])
def test_window_append_matches_oracle(gpu_lib, dtype, sink, win):
    c, appends = _case(dtype, 2, 8, seed=91, sink=sink, win=win, poison=True)
    for step, part in enumerate((0, 32)):
        app = appends if step == 0 else np.ones(len(FINAL), bool)
        log(f"window append {dtype} sink {sink} window {win} step {step} partition {part}")
        got = c.decode_append_step(seed=92 + step, appends=app, partition_tokens=part, window=(sink, win))
        _check(c, got, sink, win, f"{dtype} sink {sink} window {win} step {step}")


@pytest.mark.parametrize("H,h_q", [(1, 32), (2, 40), (4, 16), (8, 32)])
def test_window_append_group_sizes(gpu_lib, H, h_q):
    """MQA, query-head groups wider than 16, and four and eight kv heads."""
    log(f"window append H {H} h_q {h_q}")
    c, appends = _case("bf16", H, h_q, seed=93, sink=4, win=50, poison=True)
    got = c.decode_append_step(seed=94, appends=appends, window=(4, 50))
    _check(c, got, 4, 50, f"H={H} h_q={h_q}")


def test_window_append_equals_two_calls(gpu_lib):
    """The fused bf16 step leaves the same cache bits as kv_append and gives
    the output of kv_append + paged_attention_decode_window within the bf16
    bound."""
    sink, win = 4, 100
    fused, appends = _case("bf16", 8, 32, seed=95, sink=sink, win=win, poison=False)
    twin, _ = _case("bf16", 8, 32, seed=95, sink=sink, win=win, poison=False)
    got = fused.decode_append_step(seed=96, appends=appends, window=(sink, win))
    B = len(FINAL)
    new_slots = twin.pool.batch_reserve(twin.table, twin.lens, appends.astype(np.int32))
    slots = np.full(B, -1, np.int32)
    slots[appends] = new_slots
    assert np.array_equal(twin.table, fused.table)
    rng = synth.streams(96)
    k = synth.normal_bf16_bits(rng["append"], (B, 8, 128))
    v = synth.normal_bf16_bits(rng["append"], (B, 8, 128))
    twin.pool.append(0, to_dev_bits(k, "bf16"), to_dev_bits(v, "bf16"), torch.from_numpy(slots).to(DEV))
    twin.sync_tables()
    q = to_dev_bits(twin.q, "bf16")
    two = twin.pool.decode_window(0, q, twin.d_table, twin.d_lens, int(twin.lens.max()), 1.0 / math.sqrt(128),
                                  sink, win)
    torch.cuda.synchronize()
    assert torch.equal(fused.pool.k_cache.view(torch.int16), twin.pool.k_cache.view(torch.int16))
    assert torch.equal(fused.pool.v_cache.view(torch.int16), twin.pool.v_cache.view(torch.int16))
    two = oracle.bf16_bits_to_f64(two.view(torch.int16).cpu().numpy().view(np.uint16))
    assert_close(got, two, "bf16", "fused vs two calls")


def test_window_append_argument_errors(gpu_lib):
    import paged_kv_cache_271_amd as pk
    c, _ = _case("bf16", 2, 4, seed=97, sink=4, win=16, poison=False)
    B = len(FINAL)
    q = to_dev_bits(c.q, "bf16")
    kn = torch.zeros((B, 2, 128), dtype=torch.bfloat16, device=DEV)
    slots = torch.full((B,), -1, dtype=torch.int32, device=DEV)
    ml = int(c.lens.max())
    for sink, win in ((-1, 16), (4, 0)):
        with pytest.raises(pk.KVError):
            c.pool.decode_window_append(0, q, kn, kn, slots, c.d_table, c.d_lens, ml, 0.1, sink, win)
    with pytest.raises(pk.KVError):   # layer out of range
        c.pool.decode_window_append(1, q, kn, kn, slots, c.d_table, c.d_lens, ml, 0.1, 4, 16)
    with pytest.raises(ValueError):   # k_new of the wrong size
        c.pool.decode_window_append(0, q, kn[:1], kn, slots, c.d_table, c.d_lens, ml, 0.1, 4, 16)
    # no request appends: the plain windowed decode, bit for bit
    out = c.pool.decode_window_append(0, q, kn, kn, slots, c.d_table, c.d_lens, ml, 0.1, 4, 16)
    plain = c.pool.decode_window(0, q, c.d_table, c.d_lens, ml, 0.1, 4, 16)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), plain.view(torch.int16))


def test_llama3_8b_window_full_size(gpu_lib):
    """The benchmark's windowed step at full size: 64 requests of 8k-16k
    tokens with Llama-3-8B heads, 4 sinks and a 4096-token window, the dead
    pages released, then one fused step in both work splits (one token
    appended per request by the first).  Every output of twelve sampled
    requests against the oracle over the read positions; every output finite;
    the cache bits at the new slots checked by the step."""
    w = synth.WORKLOADS["llama3_8b_window"]
    sink, win = w["sink"], w["window"]
    rng = synth.streams(6)
    lens = synth.uniform_contexts(rng["contexts"], w["batch"], *w["ctx_range"])
    N = int(sum(oracle.blocks_for(int(n), 16) for n in lens))
    log(f"llama3_8b_window: B={len(lens)} ctx {lens.min()}..{lens.max()} blocks {N}")
    c = Case("bf16", w["h_kv"], w["head_dim"], w["h_q"], lens - 1, num_blocks=N,
             order=synth.permutation(rng["free_order"], N), seed=6, device_inputs=True, max_blocks=1024)
    n_rel = c.pool.window_release(c.table, c.lens, sink, win)
    assert n_rel == sum(len(oracle.dead_pages(int(n) - 1, sink, win)) for n in lens)
    c.sync_tables()
    picks = sorted(int(b) for b in rng["q"].choice(len(lens), 12, replace=False))
    for step, part in enumerate((0, w["partition_tokens"])):
        app = np.ones(len(lens), bool) if step == 0 else np.zeros(len(lens), bool)
        log(f"  fused windowed step, partition_tokens {part}")
        got = c.decode_append_step(seed=61 + step, appends=app, partition_tokens=part, window=(sink, win))
        assert c.lens_list == [int(x) for x in lens]
        _check_sampled(c, got, sink, win, picks, f"partition {part}")


def _check_sampled(c, got, sink, win, picks, what):
    q = c.q_f64()
    scale = 1.0 / math.sqrt(c.D)
    assert np.all(np.isfinite(got)), what
    for b in picks:
        K, V = c.seq_f64(b)
        ref = oracle.attention_window_fp64(q[b], K, V, scale, sink, win)
        assert_close(got[b], ref, c.tol_key, f"{what} request {b} ctx {c.lens_list[b]}")
