"""GPU parity of prefix sharing: kv_block_copy bit for bit, a forked request
writing through copy-on-write (the copy's owner sees its own tokens, every
other request's pages keep their bytes, outputs match the oracle), and a
request served from the prefix cache decoding exactly like one that computed
its own pages."""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.prefix_cache import RefPrefixCache, reserve_cow
import synth
from gpu_cases import DEV, assert_close, check_indices, check_slots, from_dev_bits, log, to_dev_bits
import paged_kv_cache_271_amd as pk

pytestmark = pytest.mark.gpu


def pool_bytes(pool):
    out = [pool.k_cache.view(torch.uint8).cpu().numpy().copy(), pool.v_cache.view(torch.uint8).cpu().numpy().copy()]
    if pool.k_scale is not None:
        out += [pool.k_scale.cpu().numpy().copy(), pool.v_scale.cpu().numpy().copy()]
    return out


def ref_bytes(ref):
    out = [ref.K.reshape(-1).view(np.uint8), ref.V.reshape(-1).view(np.uint8)]
    if ref.dtype in ("fp8", "int8"):
        out += [ref.Ks, ref.Vs]
    return out


def same(pool, ref):
    got = pool_bytes(pool)
    want = ref_bytes(ref)
    for g, w in zip(got, want):
        assert np.array_equal(g.reshape(-1).view(np.uint8), np.ascontiguousarray(w).reshape(-1).view(np.uint8))


def draw(rng, dtype, shape):
    if dtype == "f32":
        return synth.normal_f32(rng, shape)
    return synth.normal_bf16_bits(rng, shape, 0.05 if dtype in ("fp8", "int8") else 0.0, 8.0)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32", "int8"])
def test_block_copy_bit_exact(gpu_lib, dtype):
    L, N, H, D = 3, 20, 2, 128 if dtype != "f32" else 64
    rng = np.random.default_rng(41)
    pool = pk.Pool(L, N, H, D, dtype, DEV)
    ref = oracle.RefPool(L, N, H, D, 16, dtype)
    # random bytes everywhere (scales too), so every copied byte is checked
    kb = rng.integers(0, 256, tuple(pool.k_cache.view(torch.uint8).shape), dtype=np.uint8)
    vb = rng.integers(0, 256, tuple(pool.v_cache.view(torch.uint8).shape), dtype=np.uint8)
    pool.k_cache.view(torch.uint8).copy_(torch.from_numpy(kb))
    pool.v_cache.view(torch.uint8).copy_(torch.from_numpy(vb))
    ref.K = kb.reshape(-1).view(ref.K.dtype).reshape(ref.K.shape).copy()
    ref.V = vb.reshape(-1).view(ref.V.dtype).reshape(ref.V.shape).copy()
    if dtype in ("fp8", "int8"):
        ks = rng.random((L, N, H), dtype=np.float32)
        vs = rng.random((L, N, H), dtype=np.float32)
        pool.k_scale.copy_(torch.from_numpy(ks))
        pool.v_scale.copy_(torch.from_numpy(vs))
        ref.Ks, ref.Vs = ks.copy(), vs.copy()
    src = np.array([3, 7, 11, 0, 5, 99, 4], np.int32)     # 99: out of range, skipped
    dst = np.array([12, 8, 2, 19, 13, 1, 4], np.int32)    # 4 -> 4: skipped
    pool.block_copy(torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV))
    torch.cuda.synchronize()
    ref.copy_pages(src, dst)
    same(pool, ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32", "int8"])
def test_fork_copy_on_write_decode(gpu_lib, dtype):
    """A parent of 37 tokens forked into three children; every request then
    appends its own tokens for three steps through copy-on-write.  The pool
    matches the oracle pool byte for byte after every step (so the parent's
    pages never change under a child's write), and each request's decode
    matches the oracle over its own sequence."""
    H, D, h_q = 2, 128, 8
    N, MB, B = 24, 8, 4
    rng = np.random.default_rng(43)
    order = rng.permutation(N)
    pool = pk.Pool(1, N, H, D, dtype, DEV, initial_free_order=order)
    ref = oracle.RefPool(1, N, H, D, 16, dtype)
    alloc = oracle.RefAllocator(N, order)
    table = np.full((B, MB), 0, np.int32)
    lens = np.zeros(B, np.int32)
    # the parent's prefill
    slots = pool.batch_reserve(table[:1], lens[:1], np.array([37], np.int32))
    rows = [[alloc.alloc() for _ in range(3)]]
    assert list(table[0, :3]) == rows[0]
    seqs = [draw(rng, dtype, (37, H, D)), draw(rng, dtype, (37, H, D))]
    pool.append(0, to_dev_bits(seqs[0], dtype), to_dev_bits(seqs[1], dtype), torch.from_numpy(slots).to(DEV))
    ref.append(0, seqs[0], seqs[1], slots)
    kseq, vseq = [seqs[0]], [seqs[1]]
    # forks: copy the row, retain its pages
    for r in range(1, B):
        table[r] = table[0]
        lens[r] = lens[0]
        pool.retain_n(table[0, :3])
        for b in rows[0]:
            alloc.retain(b)
        rows.append(list(rows[0]))
        kseq.append(seqs[0].copy())
        vseq.append(seqs[1].copy())
    q = draw(rng, "f32" if dtype == "f32" else "bf16", (B, h_q, D))
    scale = 1.0 / math.sqrt(D)
    for step, n_new in enumerate(([0, 1, 5, 20], [2, 1, 0, 3], [1, 1, 1, 1])):
        n_new = np.array(n_new, np.int32)
        ref_lens = [int(x) for x in lens]
        want_slots, want_copies = reserve_cow(alloc, rows, ref_lens, [int(x) for x in n_new])
        s, src, dst = pool.batch_reserve_cow(table, lens, n_new)
        assert list(s) == want_slots and list(zip(src.tolist(), dst.tolist())) == want_copies
        check_slots(s, N)
        if step == 0:
            assert len(src) == 3      # every writing child copied the shared page
        if len(src):
            pool.block_copy(torch.from_numpy(src).to(DEV), torch.from_numpy(dst).to(DEV))
            for a, b in zip(src, dst):
                ref.K[:, b] = ref.K[:, a]
                ref.V[:, b] = ref.V[:, a]
                if dtype in ("fp8", "int8"):
                    ref.Ks[:, b] = ref.Ks[:, a]
                    ref.Vs[:, b] = ref.Vs[:, a]
        T = int(n_new.sum())
        k = draw(rng, dtype, (T, H, D))
        v = draw(rng, dtype, (T, H, D))
        if T:
            pool.append(0, to_dev_bits(k, dtype), to_dev_bits(v, dtype), torch.from_numpy(s).to(DEV))
            ref.append(0, k, v, s)
        o = 0
        for r in range(B):
            kseq[r] = np.concatenate([kseq[r], k[o:o + n_new[r]]])
            vseq[r] = np.concatenate([vseq[r], v[o:o + n_new[r]]])
            o += n_new[r]
        torch.cuda.synchronize()
        same(pool, ref)
        check_indices(table, lens, N, int(lens.max()))
        out = pool.decode(0, to_dev_bits(q, dtype), torch.from_numpy(table).to(DEV),
                          torch.from_numpy(lens).to(DEV), int(lens.max()), scale)
        torch.cuda.synchronize()
        got = from_dev_bits(out)
        got = got.astype(np.float64) if dtype == "f32" else oracle.bf16_bits_to_f64(got)
        qf = q.astype(np.float64) if dtype == "f32" else oracle.bf16_bits_to_f64(q)
        for r in range(B):
            K, V = ref.gather_f64(0, table[r], int(lens[r]))
            if dtype in ("bf16", "f32"):   # the stored values are the request's own inputs
                K0 = kseq[r].astype(np.float64) if dtype == "f32" else oracle.bf16_bits_to_f64(kseq[r])
                assert np.array_equal(K, K0)
            ref_o = oracle.attention_fp64(qf[r], K, V, scale)
            assert_close(got[r], ref_o, "fp8q" if dtype == "fp8" else dtype,
                         f"{dtype} step {step} request {r} (ctx {lens[r]})")


def test_prefix_cache_served_request_decodes_like_own_pages(gpu_lib):
    """Request A computes a 50-token prompt and enters its 3 whole pages in the
    cache.  Request B shares 48 tokens: its first 3 pages come from the cache,
    its tail is its own.  A twin request C computes the same tokens into
    pages of its own; B and C give the same output bits, and the oracle's."""
    H, D, h_q, N, MB = 2, 128, 8, 32, 8
    rng = np.random.default_rng(47)
    pool = pk.Pool(1, N, H, D, "bf16", DEV)
    toks_a = list(range(1000, 1050))
    toks_b = toks_a[:48] + [7, 8, 9, 10, 11]
    ka, va = draw(rng, "bf16", (50, H, D)), draw(rng, "bf16", (50, H, D))
    kt, vt = draw(rng, "bf16", (5, H, D)), draw(rng, "bf16", (5, H, D))
    table = np.zeros((3, MB), np.int32)
    lens = np.zeros(3, np.int32)
    # A: prefill, then cache its whole pages
    sa = pool.batch_reserve(table[0:1], lens[0:1], np.array([50], np.int32))
    pool.append(0, to_dev_bits(ka, "bf16"), to_dev_bits(va, "bf16"), torch.from_numpy(sa).to(DEV))
    assert pool.prefix_insert(0, toks_a, table[0, :4]) == 3
    # B: three pages from the cache, then its own 5 tokens
    hit = pool.prefix_match(0, toks_b)
    assert list(hit) == list(table[0, :3])
    assert pool.prefix_match(1, toks_b).size == 0      # another tenant: nothing
    table[1, :3] = hit
    lens[1] = 48
    sb = pool.batch_reserve(table[1:2], lens[1:2], np.array([5], np.int32))
    pool.append(0, to_dev_bits(kt, "bf16"), to_dev_bits(vt, "bf16"), torch.from_numpy(sb).to(DEV))
    # C: the same 53 tokens in pages of its own
    sc = pool.batch_reserve(table[2:3], lens[2:3], np.array([53], np.int32))
    kc = np.concatenate([ka[:48], kt])
    vc = np.concatenate([va[:48], vt])
    pool.append(0, to_dev_bits(kc, "bf16"), to_dev_bits(vc, "bf16"), torch.from_numpy(sc).to(DEV))
    for blk in hit:
        assert pool.refcount(int(blk)) == 3      # A, B and the cache
    check_indices(table, lens, N, 53)
    q1 = draw(rng, "bf16", (1, h_q, D))
    o = {}
    for r in (1, 2):    # each alone, so both see the same work split
        out = pool.decode(0, to_dev_bits(q1, "bf16"), torch.from_numpy(table[r:r + 1].copy()).to(DEV),
                          torch.from_numpy(lens[r:r + 1].copy()).to(DEV), 53, 1 / math.sqrt(D))
        torch.cuda.synchronize()
        o[r] = from_dev_bits(out)[0]
    assert np.array_equal(o[1], o[2])
    ref = oracle.attention_fp64(oracle.bf16_bits_to_f64(q1[0]), oracle.bf16_bits_to_f64(kc),
                                oracle.bf16_bits_to_f64(vc), 1 / math.sqrt(D))
    assert_close(oracle.bf16_bits_to_f64(o[1]), ref, "bf16", "cache-served request")
    log("prefix-served request matches its own-page twin bit for bit")
