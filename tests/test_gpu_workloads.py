"""GPU parity at the full workload sizes, in the launch configurations the
benchmark times (the balanced split, and 512-token partitions): the
Llama-3-8B-shaped batch (every output, with the step's append fused in and as
two calls), the Llama-3-70B-shaped long contexts (sampled heads), the fp8
batch with outliers stored as fp8 and as int8 (sampled requests; codes and
scales bit-exact), and 32 layers x 64 steps of prefix sharing with churn
(allocator state every step, sampled outputs at checkpoints)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
import workloads
from gpu_cases import Case, DEV, TOL, assert_close, check_indices, log

pytestmark = pytest.mark.gpu


def _blocks(lens):
    return int(sum(oracle.blocks_for(int(n), 16) for n in lens))


def _check_all(got, ref, what):
    worst = 0.0
    atol, rtol = TOL["bf16"]
    for b in range(len(ref)):
        err = np.abs(got[b] - ref[b])
        assert np.all(err <= atol + rtol * np.abs(ref[b])), f"{what}, request {b}: {err.max():.3e}"
        worst = max(worst, float(err.max()))
    log(f"  {what}: all {len(ref)} requests within tolerance; max|err| {worst:.3e}")


def test_llama3_8b_batch_all_outputs(gpu_lib):
    """Prefill ctx - 1 tokens, then the fused step appends the last one and
    decodes (the benchmark's step); the plain decode of the same cache in
    both splits."""
    w = synth.WORKLOADS["llama3_8b"]
    rng = synth.streams(2)
    lens = synth.uniform_contexts(rng["contexts"], w["batch"], *w["ctx_range"])
    N = _blocks(lens)
    log(f"llama3_8b: B={len(lens)} ctx {lens.min()}..{lens.max()} sum {lens.sum()} blocks {N}")
    c = Case("bf16", w["h_kv"], w["head_dim"], w["h_q"], lens - 1, num_blocks=N,
             order=synth.permutation(rng["free_order"], N), seed=2, device_inputs=True,
             max_blocks=256)
    got = c.decode_append_step(seed=21, partition_tokens=0)
    assert c.lens_list == [int(x) for x in lens]
    ref = c.oracle()
    _check_all(got, ref, "fused append + balanced decode")
    for part in (0, w["partition_tokens"]):
        _check_all(c.decode(partition_tokens=part), ref, f"decode, partition_tokens {part}")


def test_llama3_70b_long_context_sampled(gpu_lib):
    w = synth.WORKLOADS["llama3_70b_long"]
    lens = np.array(w["contexts"])
    N = _blocks(lens)
    rng = synth.streams(3)
    log(f"llama3_70b_long: ctx {lens.tolist()} blocks {N}")
    c = Case("bf16", w["h_kv"], w["head_dim"], w["h_q"], lens, num_blocks=N,
             order=synth.permutation(rng["free_order"], N), seed=3, device_inputs=True,
             max_blocks=8192)
    got = {part: c.decode(partition_tokens=part) for part in (0, w["partition_tokens"])}
    G = w["h_q"] // w["h_kv"]
    for b in range(len(lens)):
        heads = sorted(int(g * G + rng["q"].integers(0, G)) for g in rng["q"].choice(8, 3, replace=False))
        ref = c.oracle(batch=[b], heads=heads)[b]
        for part, o in got.items():
            assert_close(o[b][heads], ref, "bf16", f"ctx {lens[b]} heads {heads} partition {part}")


@pytest.mark.parametrize("dtype", ["fp8", "int8"])
def test_quantised_batch_sampled(gpu_lib, dtype):
    """The fp8 workload's batch (128 requests of 1k-8k tokens, 1% x8
    outliers), stored as fp8 E4M3 or as int8."""
    w = synth.WORKLOADS["fp8"]
    rng = synth.streams(5)
    lens = synth.uniform_contexts(rng["contexts"], w["batch"], *w["ctx_range"])
    N = _blocks(lens)
    log(f"{dtype}: B={len(lens)} ctx {lens.min()}..{lens.max()} blocks {N}")
    c = Case(dtype, w["h_kv"], w["head_dim"], w["h_q"], lens, num_blocks=N,
             order=synth.permutation(rng["free_order"], N), seed=5, device_inputs=True,
             max_blocks=512, outlier_p=w["outlier_p"], mirror=False)
    got = {part: c.decode(partition_tokens=part) for part in (0, w["partition_tokens"])}
    kc = c.pool.k_cache[0]
    vc = c.pool.v_cache[0]
    ks = c.pool.k_scale[0].cpu().numpy()
    vs = c.pool.v_scale[0].cpu().numpy()
    q = c.q_f64()
    scale = 1.0 / math.sqrt(w["head_dim"])
    for b in [int(x) for x in rng["q"].choice(len(lens), 5, replace=False)] + [int(np.argmax(lens))]:
        n = int(lens[b])
        nb = oracle.blocks_for(n, 16)
        kraw, vraw = c.seq_raw(b)
        ref_pool = oracle.RefPool(1, nb, w["h_kv"], w["head_dim"], 16, dtype)
        ref_pool.append(0, kraw, vraw, np.arange(n))
        phys = c.table[b, :nb].astype(np.int64)
        idx = torch.from_numpy(phys).to(DEV)
        assert np.array_equal(kc[idx].cpu().numpy(), ref_pool.K[0]), f"K codes of request {b}"
        assert np.array_equal(vc[idx].cpu().numpy(), ref_pool.V[0]), f"V codes of request {b}"
        assert np.array_equal(ks[phys], ref_pool.Ks[0]) and np.array_equal(vs[phys], ref_pool.Vs[0])
        Kq, Vq = ref_pool.gather_f64(0, np.arange(nb), n)
        ref_q = oracle.attention_fp64(q[b], Kq, Vq, scale)
        for part, o in got.items():
            for key in (("fp8", "fp8q") if dtype == "fp8" else ("int8",)):
                assert_close(o[b], ref_q, key, f"request {b} (ctx {n}) partition {part} vs the cached values")
        # diagnostic only: what the 8-bit storage itself costs against the inputs
        K0, V0 = oracle.bf16_bits_to_f64(kraw), oracle.bf16_bits_to_f64(vraw)
        ref0 = oracle.attention_fp64(q[b], K0, V0, scale)
        log(f"  request {b}: quantisation effect max|oracle(codes) - oracle(inputs)| "
            f"{np.max(np.abs(ref_q - ref0)):.3e}, kernel vs inputs {np.max(np.abs(got[0][b] - ref0)):.3e}")


def test_prefix_sharing_with_churn(gpu_lib):
    w = synth.WORKLOADS["prefix_churn"]
    slots = (0, 37, 101, 158, 211, 255)
    layers = (0, w["num_layers"] - 1)
    checks = {0, 1, w["steps"] // 2 - 1, w["steps"] - 1}
    ref_alloc = oracle.RefAllocator(1)
    run = workloads.PrefixChurn(DEV, layers=w["num_layers"], batch=w["batch"],
                                prefix=w["prefix_tokens"], suffix=w["suffix_range"],
                                steps=w["steps"], churn=w["churn"], seed=4,
                                record_layers=layers, record_slots=slots, mirror=ref_alloc,
                                mirror_cache=oracle.RefPrefixCache(ref_alloc))
    pb = w["prefix_tokens"] // 16
    scale = 1.0 / math.sqrt(128)
    for s in range(w["steps"]):
        outs = run.step(s)
        # allocator state every step: free count, prefix and suffix counts
        assert run.pool.num_free() == ref_alloc.num_free()
        for blk in run.prefix_blocks:
            assert run.pool.refcount(int(blk)) == 1 + w["batch"] == ref_alloc.refcount(int(blk))
        live = run.table[:, pb:][np.arange(run.MB - pb)[None, :] < ((run.lens[:, None] + 15) // 16 - pb)]
        assert len(np.unique(live)) == live.size
        for blk in live[:: max(1, live.size // 200)]:
            assert run.pool.refcount(int(blk)) == 1 == ref_alloc.refcount(int(blk))
        check_indices(run.table, run.lens, run.N, int(run.lens.max()))
        if s in checks:
            for layer in layers:
                qb, ob = outs[layer]
                q = oracle.bf16_bits_to_f64(qb)
                o = oracle.bf16_bits_to_f64(ob)
                for b in slots:
                    kbits, vbits = run.request_bits(layer, b)
                    assert kbits.shape[0] == run.lens[b]
                    ref = oracle.attention_fp64(q[b], oracle.bf16_bits_to_f64(kbits),
                                                oracle.bf16_bits_to_f64(vbits), scale)
                    assert_close(o[b], ref, "bf16", f"step {s} layer {layer} slot {b} ctx {run.lens[b]}")
        if s % 8 == 0:
            log(f"step {s}: free {run.pool.num_free()}, logical {run.logical_kv_bytes() / 1e9:.2f} GB, "
                f"unique {run.unique_kv_bytes() / 1e9:.3f} GB per layer")
    # retire everything and evict the cached prefix: the pool is whole again
    for b in range(w["batch"]):
        run._retire(b)
    assert run.pool.prefix_num_entries() == pb
    freed = run.pool.prefix_evict(pb + 10)
    # a chain: only its last page is a leaf, so the pages go last to first
    assert list(freed) == [int(x) for x in run.prefix_blocks[::-1]]
    assert run.pool.num_free() == run.N and run.pool.prefix_num_entries() == 0
