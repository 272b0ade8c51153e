"""GPU parity of the sliding-window decode with attention sinks against the
oracle: block edges for the sinks and the window start, windows wider than
the context, a window of one token, both work splits, and pages released by
kv_window_release then poisoned (a read of one would show as NaN).  Plus the
Llama-3-70B-shaped long contexts with a 4096-token window at full size."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import Case, DEV, NAN_BITS, assert_close, from_dev_bits, log

pytestmark = pytest.mark.gpu


def released_pages(before, after):
    return sorted({int(x) for x in before[(before != after)]})


def poison_pages(pool, pages, dtype):
    if not pages:
        return
    idx = torch.tensor(pages, dtype=torch.int64, device=DEV)
    if dtype == "bf16":
        pool.k_cache.view(torch.int16)[0, idx] = NAN_BITS["bf16"]
        pool.v_cache.view(torch.int16)[0, idx] = NAN_BITS["bf16"]
    else:
        pool.k_cache[0, idx] = NAN_BITS[dtype]
        pool.v_cache[0, idx] = NAN_BITS[dtype]
        pool.k_scale[0, idx] = float("nan")
        pool.v_scale[0, idx] = float("nan")


def check_visited(table, lens, sink, win, num_blocks):
    """Every page the windowed decode reads names a real block."""
    for b, n in enumerate(lens):
        for p in range(-(-int(n) // 16)):
            lo, hi = 16 * p, 16 * p + 16
            if any(t < sink or t >= n - win for t in range(lo, min(hi, int(n)))):
                assert 0 <= table[b, p] < num_blocks, (b, p)


def run_window_case(dtype, sink, win, lens, seed, H=2, h_q=8):
    N = sum(oracle.blocks_for(n, 16) for n in lens) + 3
    c = Case(dtype, H, 128, h_q, lens, num_blocks=N, order=np.random.default_rng(seed).permutation(N),
             seed=seed, poison=True)
    seqs = [c.seq_f64(b) for b in range(len(lens))]          # before any page goes
    q = c.q_f64()
    scale = 1.0 / math.sqrt(128)
    before = c.table.copy()
    n_rel = c.pool.window_release(c.table, c.lens, sink, win)
    pages = released_pages(before, c.table)
    assert n_rel == len(pages)
    dead = sum(len(oracle.dead_pages(int(n), sink, win)) for n in lens)
    assert n_rel == dead
    assert c.pool.num_free() == N - sum(oracle.blocks_for(n, 16) for n in lens) + n_rel
    poison_pages(c.pool, pages, dtype)
    c.sync_tables()
    check_visited(c.table, c.lens, sink, win, N)
    dq = synth_to_dev(c)
    outs = {}
    for part in (0, 32):
        out = c.pool.decode_window(0, dq, c.d_table, c.d_lens, max(lens), scale, sink, win, part)
        torch.cuda.synchronize()
        o = oracle.bf16_bits_to_f64(from_dev_bits(out))
        assert np.all(np.isfinite(o))
        outs[part] = o
        for b in range(len(lens)):
            K, V = seqs[b]
            ref = oracle.attention_window_fp64(q[b], K, V, scale, sink, win)
            assert_close(o[b], ref, c.tol_key, f"{dtype} sink {sink} window {win} part {part} ctx {lens[b]}")
    return outs


def synth_to_dev(c):
    from gpu_cases import to_dev_bits
    return c.dq if c.device_inputs else to_dev_bits(c.q, c.dtype)


LENS = [1, 15, 16, 17, 40, 100, 333, 1000, 0]


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "int8"])
@pytest.mark.parametrize("sink,win", [(0, 1), (4, 16), (4, 100), (17, 33), (0, 5000), (40, 7), (16, 16)])
def test_window_decode_matches_oracle(gpu_lib, dtype, sink, win):
    log(f"window decode {dtype} sink {sink} window {win}")
    run_window_case(dtype, sink, win, LENS, seed=51)


def test_window_group_sizes(gpu_lib):
    """MQA, a group wider than 16 query heads, and four kv heads (the
    workgroup-cooperative split)."""
    for H, h_q in ((1, 32), (2, 40), (4, 16), (8, 32)):
        log(f"window decode H {H} h_q {h_q}")
        run_window_case("bf16", 4, 50, [300, 17, 129, 64], seed=53, H=H, h_q=h_q)


def test_window_wider_than_context_equals_full_decode(gpu_lib):
    lens = [700, 33, 1]
    c = Case("bf16", 8, 128, 32, lens, num_blocks=60, seed=55)
    from gpu_cases import to_dev_bits
    q = to_dev_bits(c.q, "bf16")
    full = c.pool.decode(0, q, c.d_table, c.d_lens, 700, 0.088)
    win = c.pool.decode_window(0, q, c.d_table, c.d_lens, 700, 0.088, 0, 700)
    torch.cuda.synchronize()
    assert torch.equal(full.view(torch.int16), win.view(torch.int16))


def test_llama3_70b_long_context_window(gpu_lib):
    """The 70B-shaped requests (32k-128k tokens, 64 query heads) with a
    4096-token window and 4 sinks, the dead pages released: sampled heads of
    every request against the oracle over the read positions."""
    w = synth.WORKLOADS["llama3_70b_long"]
    lens = np.array(w["contexts"])
    sink, win = 4, 4096
    N = int(sum(oracle.blocks_for(int(n), 16) for n in lens))
    rng = synth.streams(3)
    c = Case("bf16", w["h_kv"], w["head_dim"], w["h_q"], lens, num_blocks=N,
             order=synth.permutation(rng["free_order"], N), seed=3, device_inputs=True, max_blocks=8192)
    keep = [np.array(oracle.window_positions(int(n), sink, win)) for n in lens]
    n_rel = c.pool.window_release(c.table, c.lens, sink, win)
    assert n_rel == sum(len(oracle.dead_pages(int(n), sink, win)) for n in lens)
    c.sync_tables()
    check_visited(c.table, c.lens, sink, win, N)
    scale = 1.0 / math.sqrt(128)
    q = c.q_f64()
    G = w["h_q"] // w["h_kv"]
    for part in (0, w["partition_tokens"]):
        out = c.pool.decode_window(0, c.dq, c.d_table, c.d_lens, int(lens.max()), scale, sink, win, part)
        torch.cuda.synchronize()
        o = oracle.bf16_bits_to_f64(from_dev_bits(out))
        for b in range(len(lens)):
            s, e = int(c.starts[b]), int(c.starts[b + 1])
            K = oracle.bf16_bits_to_f64(from_dev_bits(c.dk[s:e][torch.from_numpy(keep[b]).to(DEV)]))
            V = oracle.bf16_bits_to_f64(from_dev_bits(c.dv[s:e][torch.from_numpy(keep[b]).to(DEV)]))
            heads = sorted(int(g * G + rng["q"].integers(0, G)) for g in rng["q"].choice(8, 3, replace=False))
            for h in heads:
                g = h // G
                ref = oracle.attention_fp64(q[b][h:h + 1], K[:, g:g + 1], V[:, g:g + 1], scale)[0]
                assert_close(o[b][h], ref, "bf16", f"ctx {lens[b]} head {h} partition {part}")
