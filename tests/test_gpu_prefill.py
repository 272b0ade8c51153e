"""GPU parity of paged_attention_prefill (causal attention of each request's
new tokens over its paged cache) against the fp64 oracle: ragged prompts,
cached prefixes before the new tokens, page and tile edges, group sizes from
MHA to 128 query heads per kv head, a NaN-poisoned pool, and Llama-3-8B-shaped
2048-token prompts at full size (sampled rows)."""

import math

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_cases import DEV, NAN_BITS, assert_close, check_indices, from_dev_bits, log, to_dev_bits
import paged_kv_cache_271_amd as pk

pytestmark = pytest.mark.gpu


class PrefillCase:
    """Requests with ctx cached tokens, the last n_q of them new (queries)."""

    def __init__(self, H, D, h_q, ctx, n_q, seed, poison=False, device_inputs=False):
        self.H, self.D, self.h_q = H, D, h_q
        self.ctx = np.array(ctx, np.int32)
        self.n_q = np.array(n_q, np.int32)
        assert np.all(self.n_q <= self.ctx)
        B = len(ctx)
        N = int(sum(oracle.blocks_for(int(n), 16) for n in ctx)) + 2
        MB = max(1, max(oracle.blocks_for(int(n), 16) for n in ctx))
        rng = synth.streams(seed)
        self.pool = pk.Pool(1, N, H, D, "bf16", DEV, initial_free_order=synth.permutation(rng["free_order"], N))
        if poison:
            self.pool.k_cache.view(torch.int16).fill_(NAN_BITS["bf16"])
            self.pool.v_cache.view(torch.int16).fill_(NAN_BITS["bf16"])
        self.table = np.zeros((B, MB), np.int32)
        lens = np.zeros(B, np.int32)
        slots = self.pool.batch_reserve(self.table, lens, self.ctx)
        T = len(slots)
        self.device_inputs = device_inputs
        if device_inputs:
            self.dk = synth.device_normal((T, H, D), seed * 16 + 1, DEV, torch.bfloat16)
            self.dv = synth.device_normal((T, H, D), seed * 16 + 2, DEV, torch.bfloat16)
            self.dq = synth.device_normal((int(self.n_q.sum()), h_q, D), seed * 16 + 3, DEV, torch.bfloat16)
        else:
            self.k = synth.normal_bf16_bits(rng["k"], (T, H, D))
            self.v = synth.normal_bf16_bits(rng["v"], (T, H, D))
            self.q = synth.normal_bf16_bits(rng["q"], (int(self.n_q.sum()), h_q, D))
            self.dk, self.dv, self.dq = (to_dev_bits(x, "bf16") for x in (self.k, self.v, self.q))
        self.pool.append(0, self.dk, self.dv, torch.from_numpy(slots).to(DEV))
        self.kstart = np.concatenate([[0], np.cumsum(self.ctx)]).astype(np.int64)
        self.qstart = np.concatenate([[0], np.cumsum(self.n_q)]).astype(np.int32)
        check_indices(self.table, self.ctx, N, int(self.ctx.max()))

    def run(self, scale=None):
        scale = 1.0 / math.sqrt(self.D) if scale is None else scale
        out = self.pool.prefill(0, self.dq, torch.from_numpy(self.table).to(DEV),
                                torch.from_numpy(self.ctx).to(DEV), torch.from_numpy(self.qstart).to(DEV),
                                int(self.n_q.max()), int(self.ctx.max()), scale)
        torch.cuda.synchronize()
        return oracle.bf16_bits_to_f64(from_dev_bits(out)), scale

    def ref(self, b, rows=None, scale=None):
        s, e = int(self.kstart[b]), int(self.kstart[b + 1])
        qs, qe = int(self.qstart[b]), int(self.qstart[b + 1])
        K = oracle.bf16_bits_to_f64(from_dev_bits(self.dk[s:e]))
        V = oracle.bf16_bits_to_f64(from_dev_bits(self.dv[s:e]))
        q = oracle.bf16_bits_to_f64(from_dev_bits(self.dq[qs:qe]))
        scale = 1.0 / math.sqrt(self.D) if scale is None else scale
        if rows is None:
            return oracle.prefill_attention_fp64(q, K, V, scale)
        n, P = len(K), len(q)
        return np.stack([oracle.attention_fp64(q[i], K[:n - P + i + 1], V[:n - P + i + 1], scale) for i in rows])


CTX = [1, 16, 17, 40, 100, 300, 65, 130, 64, 1]
NQ = [1, 16, 17, 10, 64, 129, 1, 70, 64, 1]


@pytest.mark.parametrize("D", [128, 64])
def test_prefill_ragged_matches_oracle(gpu_lib, D):
    c = PrefillCase(2, D, 8, CTX, NQ, seed=61)
    got, _ = c.run()
    for b in range(len(CTX)):
        qs, qe = int(c.qstart[b]), int(c.qstart[b + 1])
        assert_close(got[qs:qe], c.ref(b), "bf16", f"D {D} ctx {CTX[b]} new {NQ[b]}")


@pytest.mark.parametrize("H,h_q", [(4, 4), (1, 8), (2, 40), (1, 64), (8, 32), (1, 128)])
def test_prefill_group_sizes(gpu_lib, H, h_q):
    """MHA (128 tokens a tile), G 8, 20 (6 tokens, 120 rows a tile), 64 (two
    tokens a tile), the Llama-3-8B ratio, and 128 (one token a tile)."""
    c = PrefillCase(H, 128, h_q, [200, 33, 7], [150, 33, 3], seed=63)
    got, _ = c.run()
    for b in range(3):
        qs, qe = int(c.qstart[b]), int(c.qstart[b + 1])
        assert_close(got[qs:qe], c.ref(b), "bf16", f"H {H} h_q {h_q} request {b}")


def test_prefill_poisoned_pool(gpu_lib):
    """Unwritten slots (the tails of last pages) hold NaN: nothing past a
    request's context reaches its output."""
    c = PrefillCase(2, 128, 8, CTX, NQ, seed=65, poison=True)
    got, _ = c.run()
    assert np.all(np.isfinite(got))
    for b in range(len(CTX)):
        qs, qe = int(c.qstart[b]), int(c.qstart[b + 1])
        assert_close(got[qs:qe], c.ref(b), "bf16", f"poisoned ctx {CTX[b]}")


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.02])
def test_prefill_any_scale(gpu_lib, scale):
    """Negative, zero and small score scales (the kernel takes maxima of raw
    scores and applies a positive scale in the exponent; the host negates q
    for a negative one)."""
    c = PrefillCase(2, 128, 8, CTX, NQ, seed=66)
    got, _ = c.run(scale)
    for b in range(len(CTX)):
        qs, qe = int(c.qstart[b]), int(c.qstart[b + 1])
        assert_close(got[qs:qe], c.ref(b, scale=scale), "bf16", f"scale {scale} ctx {CTX[b]}")


def test_prefill_one_query_equals_decode(gpu_lib):
    """n_q = 1 is the decode step: the two kernels agree within the bf16 bound."""
    ctx = [700, 33, 1, 129]
    c = PrefillCase(8, 128, 32, ctx, [1] * 4, seed=67)
    got, scale = c.run()
    dec = c.pool.decode(0, c.dq, torch.from_numpy(c.table).to(DEV), torch.from_numpy(c.ctx).to(DEV), 700, scale)
    torch.cuda.synchronize()
    assert_close(got, oracle.bf16_bits_to_f64(from_dev_bits(dec)), "bf16", "prefill vs decode")


def test_llama3_8b_prompts_full_size(gpu_lib):
    """Llama-3-8B heads: three 2048-token prompts and one 512-token chunk after
    a 1536-token cached prefix; 40 sampled rows per request (first, last,
    tile edges, random)."""
    ctx, nq = [2048, 2048, 2048, 2048], [2048, 2048, 2048, 512]
    c = PrefillCase(8, 128, 32, ctx, nq, seed=69, device_inputs=True)
    got, _ = c.run()
    rng = np.random.default_rng(69)
    for b in range(4):
        P = nq[b]
        rows = sorted({0, 1, 3, 4, P - 1, P - 2, 1023, 1024} & set(range(P)) | set(rng.integers(0, P, 32).tolist()))
        qs = int(c.qstart[b])
        ref = c.ref(b, rows)
        assert_close(got[qs + np.array(rows)], ref, "bf16", f"request {b}: {len(rows)} rows")
    log(f"prefill FLOP: {oracle.prefill_flops(ctx, nq, 32, 128) / 1e9:.1f} G")


@pytest.mark.parametrize("seed", range(8))
def test_prefill_random_shapes(gpu_lib, seed):
    """Seeded random batches: 1-6 requests, contexts 1-700 with 1..ctx new
    tokens, groups of 1-32 query heads per kv head, head_dim 64 or 128."""
    rng = np.random.default_rng(1000 + seed)
    B = int(rng.integers(1, 7))
    ctx = [int(x) for x in rng.integers(1, 701, B)]
    nq = [int(rng.integers(1, n + 1)) for n in ctx]
    H = int(rng.choice([1, 2, 4, 8]))
    G = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
    D = int(rng.choice([64, 128]))
    c = PrefillCase(H, D, H * G, ctx, nq, seed=2000 + seed)
    got, _ = c.run()
    for b in range(B):
        qs, qe = int(c.qstart[b]), int(c.qstart[b + 1])
        assert_close(got[qs:qe], c.ref(b), "bf16", f"B {B} H {H} G {G} D {D} ctx {ctx[b]} new {nq[b]}")
