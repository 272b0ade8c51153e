"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle:
append bit-exactness, decode attention on the tiny fp32 workload, special
cases, poisoned slots, physical permutation, sharing, determinism and split-K.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import Case, DEV, assert_close, check_slots, from_dev_bits, log, to_dev_bits
import paged_kv_cache_271_amd as pk

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------- append -------
def _run_slots(rng, N, T):
    """Slots shaped like request appends: runs of positions of requests whose
    pages are random blocks (partial first and last pages, a request
    continuing into the physically next block, single tokens), a few -1
    entries.  No slot repeats."""
    free = list(rng.permutation(N))
    out = []
    while len(out) < T and len(free) >= 3:
        start = int(rng.integers(0, 16))
        n = int(rng.integers(1, 48))
        pages = [free.pop(), free.pop(), free.pop()]
        if rng.random() < 0.3 and pages[0] + 1 < N and (pages[0] + 1) in free:
            free.remove(pages[0] + 1)
            pages[1] = pages[0] + 1        # slots run on across a block boundary
        for pos in range(start, min(start + n, 48)):
            out.append(pages[pos // 16] * 16 + pos % 16)
    out = np.array(out[:T], np.int32)
    out[rng.random(len(out)) < 0.03] = -1
    return out


@pytest.mark.parametrize("pattern", ["scattered", "runs", "bulk"])
@pytest.mark.parametrize("dtype,D", [("f32", 64), ("f32", 128), ("bf16", 128), ("bf16", 64)])
def test_append_copy_bit_exact(gpu_lib, dtype, D, pattern):
    log(f"append {dtype} D={D} {pattern}")
    H, N = 2, {"scattered": 12, "runs": 60, "bulk": 600}[pattern]
    rng = np.random.default_rng(1)
    order = rng.permutation(N)
    pool = pk.Pool(2, N, H, D, dtype, DEV, initial_free_order=order)
    ref = oracle.RefPool(2, N, H, D, 16, dtype)
    # start from a non-zero background so untouched slots are checked too
    kb, vb = pool.k_cache.view(torch.uint8), pool.v_cache.view(torch.uint8)
    bg_k = rng.integers(0, 2 ** 8, tuple(kb.shape), dtype=np.uint8)
    bg_v = rng.integers(0, 2 ** 8, tuple(vb.shape), dtype=np.uint8)
    kb.copy_(torch.from_numpy(bg_k).to(DEV))
    vb.copy_(torch.from_numpy(bg_v).to(DEV))
    ref.K = bg_k.reshape(-1).view(ref.K.dtype).reshape(ref.K.shape).copy()
    ref.V = bg_v.reshape(-1).view(ref.V.dtype).reshape(ref.V.shape).copy()
    for layer in range(2):
        for call in range(4):
            if pattern == "scattered":
                T = int(rng.integers(1, 40))
                slots = rng.choice(N * 16, T, replace=False).astype(np.int32)
                slots[rng.random(T) < 0.1] = -1
            else:   # bulk calls (over 1024 tokens) take the kernel's other launch shape
                T = int(rng.integers(1, 160)) if pattern == "runs" else int(rng.integers(1100, 3000))
                slots = _run_slots(rng, N, T)
                T = len(slots)
                assert pattern == "runs" or T > 1024
            check_slots(slots, N)
            if dtype == "f32":
                k = synth.normal_f32(rng, (T, H, D))
                v = synth.normal_f32(rng, (T, H, D))
            else:
                k = synth.normal_bf16_bits(rng, (T, H, D))
                v = synth.normal_bf16_bits(rng, (T, H, D))
            pool.append(layer, to_dev_bits(k, dtype), to_dev_bits(v, dtype),
                        torch.from_numpy(slots).to(DEV))
            ref.append(layer, k, v, slots)
    torch.cuda.synchronize()
    # compare bytes (the random background holds NaN patterns)
    assert np.array_equal(pool.k_cache.view(torch.uint8).cpu().numpy().reshape(-1), ref.K.reshape(-1).view(np.uint8))
    assert np.array_equal(pool.v_cache.view(torch.uint8).cpu().numpy().reshape(-1), ref.V.reshape(-1).view(np.uint8))


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_append_quantised_bit_exact(gpu_lib, dtype):
    log(f"append {dtype}")
    H, D, N = 3, 128, 10
    rng = np.random.default_rng(2)
    pool = pk.Pool(1, N, H, D, dtype, DEV, initial_free_order=rng.permutation(N))
    ref = oracle.RefPool(1, N, H, D, 16, dtype)
    table = np.zeros((3, 4), np.int32)
    lens = np.zeros(3, np.int32)
    # bulk fills, single tokens growing the scale, and mixed run lengths
    for n_new in ([20, 5, 0], [1, 1, 1], [3, 0, 30], [1, 12, 1], [0, 1, 0], [9, 9, 9]):
        n_new = np.array(n_new, np.int32)
        slots = pool.batch_reserve(table, lens, n_new)
        T = len(slots)
        k = synth.normal_bf16_bits(rng, (T, H, D), 0.05, 8.0)
        v = synth.normal_bf16_bits(rng, (T, H, D), 0.05, 8.0)
        # single tokens larger than before force re-encoding of earlier slots
        k = synth.f32_to_bf16_bits(oracle.bf16_bits_to_f64(k).astype(np.float32) * np.float32(rng.uniform(0.5, 3)))
        check_slots(slots, N)
        pool.append(0, to_dev_bits(k, dtype), to_dev_bits(v, dtype), torch.from_numpy(slots).to(DEV))
        ref.append(0, k, v, slots)
        torch.cuda.synchronize()
        assert np.array_equal(pool.k_scale.cpu().numpy(), ref.Ks)
        assert np.array_equal(pool.v_scale.cpu().numpy(), ref.Vs)
        assert np.array_equal(pool.k_cache.cpu().numpy(), ref.K)
        assert np.array_equal(pool.v_cache.cpu().numpy(), ref.V)


# ------------------------------------------------------- tiny fp32 case ------
def test_tiny_f32_two_steps(gpu_lib):
    """1 layer, requests of 17 and 40 tokens, h_q 4, h_kv 2, d_h 64, 16-block
    pool in a seeded random order; decode; append one token each; decode."""
    w = synth.WORKLOADS["tiny_f32"]
    rng = synth.streams(1)
    order = synth.permutation(rng["free_order"], w["pool_blocks"])
    c = Case("f32", w["h_kv"], w["head_dim"], w["h_q"], w["contexts"], num_blocks=w["pool_blocks"],
             order=order, seed=1, max_blocks=3)
    for step in range(2):
        log(f"tiny f32 step {step}: ctx {c.lens_list}")
        got = c.decode()
        ref = c.oracle()
        for b in range(2):
            assert_close(got[b], ref[b], c.tol_key, f"request {b}")
        split = c.decode(partition_tokens=16)
        assert np.max(np.abs(split - got)) <= 1e-6
        if step == 0:
            c.grow(seed=11)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "int8"])
def test_block_boundaries_and_split(gpu_lib, dtype):
    """Contexts at and around block edges, growing across them; forced small
    partitions agree with one partition."""
    lens = [1, 15, 16, 17, 31, 32, 33, 64, 100]
    c = Case(dtype, 2, 128, 8, lens, num_blocks=64, order=np.random.default_rng(5).permutation(64),
             seed=3, max_blocks=8)
    for step in range(2):
        got = c.decode()
        ref_in = c.oracle()
        for b in range(len(lens)):
            assert_close(got[b], ref_in[b], c.tol_key, f"{dtype} ctx {c.lens_list[b]}")
        for part in (16, 32, 48):
            split = c.decode(partition_tokens=part)
            assert np.max(np.abs(split - got)) <= (1e-6 if dtype == "f32" else 2e-2)
        c.grow(seed=20 + step)


# ------------------------------------------------------ special cases -------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identical_keys_give_mean_of_values(gpu_lib, dtype):
    c = Case(dtype, 2, 64, 4, [37, 5], num_blocks=8, seed=4)
    same = c.k[:1].copy()
    # rewrite every K with the same vector through the append path
    k = np.repeat(same, c.k.shape[0], axis=0)
    slots = np.concatenate([c.pool.slot_mapping(c.table[b], np.arange(n)) for b, n in enumerate(c.lens_list)])
    c.append_host(k, c.v, slots.astype(np.int32))
    got = c.decode()
    for b in range(2):
        _, V = c.seq_f64(b)
        want = np.repeat(V.mean(axis=0), 2, axis=0)
        assert_close(got[b], want, c.tol_key, f"mean of V, request {b}")


@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "int8"])
@pytest.mark.parametrize("D", [128, 64])
def test_one_token_and_empty(gpu_lib, dtype, D):
    c = Case(dtype, 2, D, 4, [1, 0, 1, 0], num_blocks=4, seed=5)
    got = c.decode(nan_out=True)     # empty requests' rows are written as zeros
    assert not np.any(got[1]) and not np.any(got[3])
    for b in (0, 2):
        _, V = c.seq_f64(b)
        want = np.repeat(V[0], 2, axis=0)
        assert_close(got[b], want, c.tol_key, f"ctx 1, request {b}")
    # all requests empty
    e = Case(dtype, 2, D, 4, [0, 0], num_blocks=2, seed=6, max_blocks=1)
    assert not np.any(e.decode(max_ctx=0, nan_out=True))


@pytest.mark.parametrize("H,h_q", [(1, 32), (4, 4), (2, 40), (1, 1)])
def test_group_sizes_mqa_mha(gpu_lib, H, h_q):
    """MQA (one KV head), MHA (G = 1) and groups wider than 16 query heads."""
    for dtype in ("bf16", "f32"):
        c = Case(dtype, H, 64, h_q, [70, 3, 129], num_blocks=20, seed=7)
        got = c.decode()
        ref = c.oracle()
        for b in range(3):
            assert_close(got[b], ref[b], c.tol_key, f"{dtype} H={H} h_q={h_q} request {b}")


@pytest.mark.parametrize("H,h_q", [(1, 32), (4, 4), (2, 40), (1, 1)])
def test_group_sizes_ring(gpu_lib, H, h_q):
    """The same group shapes at head_dim 128, where bf16, fp8 and int8 pools
    run the LDS-ring decode: waves that do not share a request when the
    kv-head groups do not come in fours, two head groups per kv head when
    G > 16; balanced and 16-token partitions."""
    for dtype in ("bf16", "fp8", "int8"):
        c = Case(dtype, H, 128, h_q, [70, 3, 129, 1000], num_blocks=80, seed=8)
        ref = c.oracle()
        for part in (0, 16):
            got = c.decode(partition_tokens=part)
            for b in range(4):
                assert_close(got[b], ref[b], c.tol_key, f"{dtype} H={H} h_q={h_q} part {part} request {b}")


# ------------------------------------------------ invariance / poison -------
@pytest.mark.parametrize("dtype", ["f32", "bf16", "fp8", "int8"])
def test_poisoned_slots_do_not_leak(gpu_lib, dtype):
    """NaN in every unwritten slot (and scale) never reaches an output.
    Partitions of 16 and 48 tokens end every segment in a one-block step,
    whose missing second block the kernel loads from the segment's last
    table entry and masks."""
    lens = [17, 40, 3, 130]
    clean = Case(dtype, 2, 128, 8, lens, num_blocks=30, seed=8, order=np.arange(30))
    dirty = Case(dtype, 2, 128, 8, lens, num_blocks=30, seed=8, order=np.arange(30), poison=True)
    for part in (0, 16, 32, 48):
        a, b = clean.decode(partition_tokens=part), dirty.decode(partition_tokens=part)
        assert np.all(np.isfinite(b)), f"partition {part}"
        assert np.array_equal(a, b), f"partition {part}"


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "f32", "int8"])
def test_physical_permutation_bit_identical(gpu_lib, dtype):
    lens = [300, 17, 1000, 64]
    N = sum(oracle.blocks_for(n, 16) for n in lens) + 7
    rng = np.random.default_rng(9)
    a = Case(dtype, 2, 128, 8, lens, num_blocks=N, seed=10, order=np.arange(N))
    b = Case(dtype, 2, 128, 8, lens, num_blocks=N, seed=10, order=rng.permutation(N))
    assert not np.array_equal(a.table, b.table)
    for part in (0, 128):
        assert np.array_equal(a.decode(partition_tokens=part), b.decode(partition_tokens=part))


@pytest.mark.parametrize("dtype", ["bf16", "fp8", "int8"])
def test_shared_prefix_equals_duplicated(gpu_lib, dtype):
    """Requests mapping one set of prefix blocks give the same bits as
    requests holding private copies."""
    H, D, h_q, pre, n_req = 2, 128, 8, 64, 3
    rng = synth.streams(12)
    suf = [5, 20, 33]
    pk_bits = synth.normal_bf16_bits(rng["k"], (pre, H, D))
    pv_bits = synth.normal_bf16_bits(rng["v"], (pre, H, D))
    sk = [synth.normal_bf16_bits(rng["k"], (n, H, D)) for n in suf]
    sv = [synth.normal_bf16_bits(rng["v"], (n, H, D)) for n in suf]
    q = synth.normal_bf16_bits(rng["q"], (n_req, h_q, D))
    outs = []
    for shared in (True, False):
        pool = pk.Pool(1, 40, H, D, dtype, DEV)
        table = np.zeros((n_req, 8), np.int32)
        lens = np.zeros(n_req, np.int32)
        if shared:
            prefix = [pool.alloc() for _ in range(pre // 16)]
            slots = pool.slot_mapping(prefix, np.arange(pre))
            pool.append(0, to_dev_bits(pk_bits, dtype), to_dev_bits(pv_bits, dtype),
                        torch.from_numpy(slots).to(DEV))
            for r in range(n_req):
                for blk in prefix:
                    pool.retain(blk)
                table[r, :len(prefix)] = prefix
                lens[r] = pre
        for r in range(n_req):
            if not shared:
                tr = table[r:r + 1]
                lr = lens[r:r + 1]
                slots = pool.batch_reserve(tr, lr, np.array([pre], np.int32))
                pool.append(0, to_dev_bits(pk_bits, dtype), to_dev_bits(pv_bits, dtype),
                            torch.from_numpy(slots).to(DEV))
            tr = table[r:r + 1]
            lr = lens[r:r + 1]
            slots = pool.batch_reserve(tr, lr, np.array([suf[r]], np.int32))
            pool.append(0, to_dev_bits(sk[r], dtype), to_dev_bits(sv[r], dtype),
                        torch.from_numpy(slots).to(DEV))
        if shared:
            assert pool.refcount(int(table[0, 0])) == 1 + n_req
        from gpu_cases import check_indices
        check_indices(table, lens, 40, 100)
        out = pool.decode(0, to_dev_bits(q, dtype), torch.from_numpy(table).to(DEV),
                          torch.from_numpy(lens).to(DEV), 100, 1 / math.sqrt(D))
        torch.cuda.synchronize()
        outs.append(from_dev_bits(out))
    assert np.array_equal(outs[0], outs[1])


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("fp8", 128), ("int8", 128)])
def test_cache_hint_bit_identical(gpu_lib, dtype, D):
    """The decode reads K/V with the non-temporal hint while no block is
    mapped twice and with plain loads otherwise (kv_num_shared_blocks).  A
    block that no table lists is retained to switch the pool over: the
    outputs stay bit-identical, balanced and fixed splits alike."""
    lens = [int(x) for x in np.random.default_rng(31).integers(1, 3000, 24)]
    need = sum(oracle.blocks_for(n, 16) for n in lens)
    c = Case(dtype, 2, D, 8, lens, num_blocks=need + 1, seed=31)
    assert c.pool.num_shared() == 0
    plain = [c.decode(partition_tokens=p) for p in (0, 64)]
    spare = c.pool.alloc()
    c.pool.retain(spare)
    assert c.pool.num_shared() == 1
    assert all(np.array_equal(a, c.decode(partition_tokens=p)) for a, p in zip(plain, (0, 64)))
    c.pool.release(spare)
    assert c.pool.num_shared() == 0


def test_deterministic_repeats(gpu_lib):
    c = Case("bf16", 8, 128, 32, [700, 2000, 33, 4096], num_blocks=600, seed=13)
    a = c.decode()
    for _ in range(3):
        assert np.array_equal(a, c.decode())


def test_balanced_split_reused_workspace(gpu_lib):
    """A 64-request batch with about 23 blocks per workgroup chunk (the split
    the benchmark runs): one workspace reused over repeated calls gives
    bit-identical outputs, sampled requests match the oracle, and a fixed
    split agrees within the bf16 bound."""
    lens = [int(x) for x in np.random.default_rng(21).integers(900, 1300, 64)]
    c = Case("bf16", 8, 128, 32, lens, seed=21, device_inputs=True)
    max_ctx = max(lens)
    ws = c.pool.new_workspace(64, 32, max_ctx)
    outs = []
    for _ in range(3):
        out = c.pool.decode(0, c.dq, c.d_table, c.d_lens, max_ctx, 1.0 / math.sqrt(128), 0, workspace=ws)
        torch.cuda.synchronize()
        outs.append(from_dev_bits(out))
    assert all(np.array_equal(outs[0], o) for o in outs[1:])
    got = oracle.bf16_bits_to_f64(outs[0])
    ref = c.oracle(batch=[0, 17, 40, 63])
    for b in (0, 17, 40, 63):
        assert_close(got[b], ref[b], "bf16", f"request {b} of {lens[b]} tokens")
    fixed = c.decode(partition_tokens=256)
    assert np.max(np.abs(fixed - got)) <= 2e-2


@pytest.mark.parametrize("dtype,B,D", [("bf16", 8192, 64), ("bf16", 8192, 128), ("bf16", 4096, 128),
                                       ("fp8", 8192, 128), ("int8", 4096, 128)])
def test_largest_batch(gpu_lib, dtype, B, D):
    """The largest batches, of 0-40 tokens per request: 8192 (the bound of
    the balanced decode) and 4096 (the bound of the LDS-ring decode, which
    pools with head_dim 128 take up to that size; larger batches fall back
    to the register-streaming decode).  The block prefix is scanned in
    many passes, chunks hold many whole requests, empty requests give zeros.
    Plain decode, then the fused step (which also appends B rows); a sample
    of requests is checked against the oracle, and every output is finite.
    8-bit pools: the register-streaming (8192) and ring (4096) decodes with
    their fused append."""
    rng = np.random.default_rng(81)
    lens = rng.integers(0, 41, B)
    lens[rng.choice(B, 200, replace=False)] = 0
    need = int(sum(oracle.blocks_for(int(n), 16) for n in lens))
    c = Case(dtype, 2, D, 8, lens, num_blocks=need + B, max_blocks=4, seed=81, mirror=dtype != "bf16")
    sample = sorted(set(rng.choice(B, 48, replace=False).tolist()) | {0, B - 1, int(np.argmax(lens))})
    got = c.decode()
    assert np.all(np.isfinite(got))
    ref = c.oracle(batch=sample)
    for b in sample:
        assert_close(got[b], ref[b], c.tol_key, f"{dtype} request {b} of {c.lens_list[b]} tokens")
    assert np.all(got[np.array(c.lens_list) == 0] == 0)
    got = c.decode_append_step(seed=82)
    ref = c.oracle(batch=sample)
    for b in sample:
        assert_close(got[b], ref[b], c.tol_key, f"{dtype} fused step, request {b} of {c.lens_list[b]} tokens")


@pytest.mark.parametrize("seed", range(8))
def test_random_shapes(gpu_lib, seed):
    """Seeded random batches for the decode: element type, kv heads, group
    size (1-20 query heads per kv head), head_dim, 1-24 requests of 0-2500
    tokens (fp8/int8: 1-8 of 0-1200), and the split (balanced, or pieces of
    16-512 tokens)."""
    rng = np.random.default_rng(3000 + seed)
    dtype = str(rng.choice(["bf16", "fp8", "int8", "f32"]))
    H = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.integers(1, 21))
    D = int(rng.choice([64, 128]))
    q8 = dtype in ("fp8", "int8")   # the oracle reads a host mirror of the quantised pool
    B = int(rng.integers(1, 9 if q8 else 25))
    lens = [int(x) for x in rng.integers(0, 1201 if q8 else 2501, B)]
    part = int(rng.choice([0, 0, 16, 64, 512]))
    c = Case(dtype, H, D, H * G, lens, seed=4000 + seed, mirror=q8)
    got = c.decode(partition_tokens=part)
    ref = c.oracle()
    for b in range(B):
        assert_close(got[b], ref[b], c.tol_key, f"{dtype} H {H} G {G} D {D} part {part} ctx {lens[b]}")
