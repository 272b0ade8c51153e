"""Pins of the oracle's memory arithmetic, block counts, allocator, slot mapping
and pool model against what the pages print and against brute force.
CPU only."""

import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- sizes ------
def test_bytes_per_token_worked_examples():
    g = _golden("kv_memory_examples.json")
    c8, c70 = g["per_token"]
    assert oracle.kv_bytes_per_token(c8["L"], c8["h_kv"], c8["d_h"], c8["b"]) == c8["bytes_per_token"]
    b70 = oracle.kv_bytes_per_token(c70["L"], c70["h_kv"], c70["d_h"], c70["b"])
    assert b70 == c70["printed_kb"] * 1024          # "320 KB" in binary kilobytes


def test_per_request_totals_round_to_printed():
    g = _golden("kv_memory_examples.json")
    for c in g["per_request"]:
        tot = oracle.kv_total_bytes(c["B"], c["T"], c["L"], c["h_kv"], c["d_h"], c["b"])
        assert round(tot / 2 ** 30) == c["printed_gb"]
    # the exact values behind "~1 GB" and "~40 GB"
    assert oracle.kv_total_bytes(1, 8192, 32, 8, 128, 2) == 2 ** 30
    assert oracle.kv_total_bytes(1, 131072, 80, 8, 128, 2) == 40 * 2 ** 30


def test_capacity_example_decimal_units():
    c = _golden("kv_memory_examples.json")["capacity"]
    tokens = c["free_bytes"] // c["bytes_per_token"]
    assert tokens == 62500 and tokens // 1000 == c["printed_k_tokens"]


def test_fp8_halves_and_per_layer_bytes():
    r = _golden("kv_memory_examples.json")["fp8"]["ratio"]
    assert oracle.kv_bytes_per_token(32, 8, 128, 1) == r * oracle.kv_bytes_per_token(32, 8, 128, 2)
    # one layer of the Llama-3-8B shape, bf16: 2 * 8 * 128 * 2
    assert oracle.kv_bytes_per_token(1, 8, 128, 2) == 4096


def test_hidden_dim_form_is_the_mha_case():
    # the glossary's form equals the per-head form when hidden = h_kv * d_h
    for L, h, d, b in [(32, 32, 128, 2), (80, 64, 128, 2), (2, 3, 5, 4)]:
        assert oracle.kv_total_bytes_hidden(3, 7, L, h * d, b) == oracle.kv_total_bytes(3, 7, L, h, d, b)
    # with GQA the two forms differ: 70B at 4096 tokens is 1.34 GB, not the
    # glossary's "over 2.5 GB"; the per-head form is the one used for sizing
    assert oracle.kv_total_bytes(1, 4096, 80, 8, 128, 2) == 1342177280


def test_sliding_window_constant_in_length():
    # 2 * W * L * d_kv * b, independent of how long the request is
    assert oracle.sliding_window_bytes(4096, 32, 8 * 128, 2) == 4096 * 131072 == 512 * 2 ** 20


def test_blocks_for_pages_example_and_bruteforce():
    p = _golden("kv_memory_examples.json")["paging"]
    assert oracle.blocks_for(p["tokens"], p["block_size"]) == p["pages"]
    assert oracle.wasted_slots(p["tokens"], p["block_size"]) == p["wasted_slots"]
    for n in range(0, 101):
        k = 0
        while 16 * k < n:
            k += 1
        assert oracle.blocks_for(n, 16) == k
        assert 0 <= oracle.wasted_slots(n, 16) < 16


# ------------------------------------------------------------ allocator ------
def test_allocator_lifo_order():
    order = [5, 2, 7, 0, 1, 3, 4, 6]
    a = oracle.RefAllocator(8, order)
    assert [a.alloc() for _ in range(3)] == [5, 2, 7]
    a.release(2)
    assert a.alloc() == 2          # last released is handed out next
    assert a.alloc() == 0
    assert a.free_list_top_first() == [1, 3, 4, 6]


def test_allocator_errors_leave_state():
    a = oracle.RefAllocator(2)
    b0, b1 = a.alloc(), a.alloc()
    with pytest.raises(oracle.NoBlocks):
        a.alloc()
    a.release(b0)
    with pytest.raises(oracle.BadBlock):
        a.release(b0)               # double release
    with pytest.raises(oracle.BadBlock):
        a.retain(b0)                # retain of a free page
    with pytest.raises(oracle.BadBlock):
        a.retain(5)
    assert a.num_free() == 1 and a.refcount(b1) == 1


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 24), seed=st.integers(0, 2 ** 31 - 1),
       ops=st.lists(st.tuples(st.sampled_from(["alloc", "retain", "release"]),
                              st.integers(0, 30)), max_size=120))
def test_allocator_against_set_model(n, seed, ops):
    """Brute-force model: a set of free ids and a dict of counts."""
    order = list(np.random.default_rng(seed).permutation(n))
    a = oracle.RefAllocator(n, order)
    free, rc = set(range(n)), {}
    for op, x in ops:
        if op == "alloc":
            if not free:
                with pytest.raises(oracle.NoBlocks):
                    a.alloc()
                continue
            b = a.alloc()
            assert b in free
            free.discard(b)
            rc[b] = 1
        else:
            b = x % (n + 3)            # sometimes out of range
            live = b in rc
            if not live:
                with pytest.raises(oracle.BadBlock):
                    getattr(a, op)(b)
                continue
            getattr(a, op)(b)
            if op == "retain":
                rc[b] += 1
            else:
                rc[b] -= 1
                if rc[b] == 0:
                    del rc[b]
                    free.add(b)
        assert a.num_free() == len(free)
        assert a.num_free() + len(rc) == n
        assert set(a.free_list_top_first()) == free
        for b in range(n):
            assert a.refcount(b) == rc.get(b, 0)


# ------------------------------------------------------------ slots, pool ----
def test_slot_closed_form_and_distinct():
    rng = np.random.default_rng(0)
    table = rng.permutation(40)[:10]
    slots = oracle.slot_mapping(table, range(150), 16)
    for p, s in enumerate(slots):
        assert s == table[p // 16] * 16 + p % 16
    assert len(set(slots.tolist())) == 150


def test_slot_mapping_refuses_shared_and_free_pages():
    a = oracle.RefAllocator(4)
    b = a.alloc()
    a.retain(b)
    with pytest.raises(oracle.SharedBlockWrite):
        oracle.slot_mapping([b], [3], 16, a.refcount)
    with pytest.raises(oracle.BadBlock):
        oracle.slot_mapping([3], [0], 16, a.refcount)


def _fill(dtype, seed, lens, H=2, D=8, nblocks=20, order=None):
    """Append tokens of several requests into a pool and into SeqKV, one
    append call per request chunk."""
    rng = np.random.default_rng(seed)
    pool = oracle.RefPool(1, nblocks, H, D, 16, dtype)
    alloc = oracle.RefAllocator(nblocks, order)
    seqs, tables = [], []
    for n in lens:
        s = oracle.SeqKV(H, D, "f32" if dtype == "f32" else "bf16")
        table = [alloc.alloc() for _ in range(oracle.blocks_for(n, 16))]
        done = 0
        while done < n:
            c = min(n - done, int(rng.integers(1, 20)))
            if dtype == "f32":
                k = synth.normal_f32(rng, (c, H, D))
                v = synth.normal_f32(rng, (c, H, D))
            else:
                k = synth.normal_bf16_bits(rng, (c, H, D))
                v = synth.normal_bf16_bits(rng, (c, H, D))
            slots = oracle.slot_mapping(table, range(done, done + c), 16)
            pool.append(0, k, v, slots)
            s.append(k, v)
            done += c
        seqs.append(s)
        tables.append(table)
    return pool, seqs, tables


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_pool_gather_reproduces_contiguous_cache(dtype):
    pool, seqs, tables = _fill(dtype, 1, [17, 40, 1, 0, 33])
    for s, t in zip(seqs, tables):
        kr, vr = pool.gather_raw(0, t, len(s))
        assert np.array_equal(kr, s.K) and np.array_equal(vr, s.V)


def test_pool_gather_invariant_under_physical_permutation():
    lens = [17, 40, 33]
    pa, sa, ta = _fill("bf16", 2, lens, order=list(range(20)))
    pb, sb, tb = _fill("bf16", 2, lens, order=list(np.random.default_rng(9).permutation(20)))
    assert sum(ta, []) != sum(tb, [])           # different physical placement
    for i, n in enumerate(lens):
        for x, y in zip(pa.gather_f64(0, ta[i], n), pb.gather_f64(0, tb[i], n)):
            assert np.array_equal(x, y)


def test_pool_layout_is_token_major_k_dim_major_v():
    pool = oracle.RefPool(1, 2, 1, 4, 16, "f32")
    k = np.arange(4, dtype=np.float32).reshape(1, 1, 4)
    pool.append(0, k, k + 10, [16 + 3])
    assert np.array_equal(pool.K[0, 1, 0, 3, :], [0, 1, 2, 3])
    assert np.array_equal(pool.V[0, 1, 0, :, 3], [10, 11, 12, 13])
    assert pool.K.sum() == 6 and pool.V.sum() == 46


def test_bf16_widening_exact():
    bits = np.array([0x3F80, 0xBF80, 0x0000, 0x8000, 0x7F7F, 0x0001, 0x4049], np.uint16)
    want = [1.0, -1.0, 0.0, -0.0, 3.3895313892515355e38, 2.0 ** -133, 3.140625]
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), np.array(want))
    # the input rounding in synth is round-to-nearest-even
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    assert synth.f32_to_bf16_bits(x).tolist() == [0x3F80, 0x3F82, 0x3F81]
