"""Seeded synthetic inputs for paged decode attention.

Shared by the tests, the benchmark and the smoke check; it holds no attention,
paging or quantisation arithmetic -- only shapes, seeded draws and the
float32 -> bfloat16 input rounding (round to nearest even), so that the HIP
library and the reference receive the identical bit patterns.

Workloads (block size 16 everywhere):

* tiny_f32 -- 1 layer, 2 requests of 17 and 40 tokens, h_q 4, h_kv 2, d_h 64,
  fp32 cache, a 16-block pool handed out in a seeded random order; then one
  more token per request.
* llama3_8b -- Llama-3-8B attention shape for one layer: h_q 32, h_kv 8,
  d_h 128, bf16, batch 64, contexts uniform on [512, 4096].
* llama3_70b_long -- Llama-3-70B shape for one layer: h_q 64, h_kv 8, d_h 128,
  bf16, batch 4 with contexts 32768, 65536, 98304, 131072, split into
  512-token partitions.
* prefix_churn -- Llama-3-8B heads, 32 layers, 256 requests sharing a
  2000-token prefix plus unique suffixes uniform on [5, 500]; 64 steps with
  26 of 256 requests retired and replaced per step.
* fp8 -- Llama-3-8B heads, fp8 E4M3 cache with per-(block, kv-head) scales,
  bf16 queries, batch 128, contexts uniform on [1024, 8192]; K/V values N(0,1)
  with each element independently multiplied by 8 with probability 0.01.

Values are N(0, 1) drawn as float32.  "Uniform on [a, b]" means integers with
both ends included.  Host draws use numpy's PCG64 generator from
``SeedSequence(seed).spawn``; large K/V inputs are drawn on the device with a
seeded ``torch.Generator`` (inputs only; the reference receives host copies of
exactly those bits).
"""

import math

import numpy as np

BLOCK_SIZE = 16

WORKLOADS = {
    "tiny_f32": dict(dtype="f32", num_layers=1, h_q=4, h_kv=2, head_dim=64,
                     batch=2, contexts=(17, 40), pool_blocks=16, steps=1,
                     partition_tokens=512),
    "llama3_8b": dict(dtype="bf16", num_layers=1, h_q=32, h_kv=8, head_dim=128,
                      batch=64, ctx_range=(512, 4096), partition_tokens=512),
    "llama3_70b_long": dict(dtype="bf16", num_layers=1, h_q=64, h_kv=8, head_dim=128,
                            batch=4, contexts=(32768, 65536, 98304, 131072),
                            partition_tokens=512),
    "prefix_churn": dict(dtype="bf16", num_layers=32, h_q=32, h_kv=8, head_dim=128,
                         batch=256, prefix_tokens=2000, suffix_range=(5, 500),
                         steps=64, churn=26, partition_tokens=512),
    "llama3_8b_window": dict(dtype="bf16", num_layers=1, h_q=32, h_kv=8, head_dim=128,
                             batch=64, ctx_range=(8192, 16384), sink=4, window=4096,
                             partition_tokens=512),
    "fp8": dict(dtype="fp8", num_layers=1, h_q=32, h_kv=8, head_dim=128,
                batch=128, ctx_range=(1024, 8192), outlier_p=0.01,
                outlier_mul=8.0, partition_tokens=512),
    # the fp8 batch stored as symmetric int8 codes
    "int8": dict(dtype="int8", num_layers=1, h_q=32, h_kv=8, head_dim=128,
                 batch=128, ctx_range=(1024, 8192), outlier_p=0.01,
                 outlier_mul=8.0, partition_tokens=512),
}

# sub-stream order of SeedSequence(seed).spawn(...)
STREAMS = ("contexts", "free_order", "q", "k", "v", "append", "churn")


def streams(seed):
    """Named numpy generators for one seed."""
    kids = np.random.SeedSequence(seed).spawn(len(STREAMS))
    return {name: np.random.Generator(np.random.PCG64(s)) for name, s in zip(STREAMS, kids)}


def f32_to_bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even
    (NaN kept quiet)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x40)).astype(np.uint16)
    return out


def normal_f32(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def normal_bf16_bits(rng, shape, outlier_p=0.0, outlier_mul=1.0):
    x = rng.standard_normal(shape, dtype=np.float32)
    if outlier_p > 0.0:
        mask = rng.random(shape, dtype=np.float32) < outlier_p
        x[mask] *= np.float32(outlier_mul)
    return f32_to_bf16_bits(x)


def uniform_contexts(rng, batch, lo, hi):
    return rng.integers(lo, hi + 1, size=batch).astype(np.int64)


def permutation(rng, n):
    return rng.permutation(n).astype(np.int64)


def blocks_needed(n_tokens):
    return (n_tokens + BLOCK_SIZE - 1) // BLOCK_SIZE


def device_normal(shape, seed, device, dtype, outlier_p=0.0, outlier_mul=1.0):
    """N(0,1) float32 drawn on `device` with a seeded torch generator, optional
    outliers, then cast to `dtype` (torch float32 -> bfloat16 rounds to
    nearest even)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if outlier_p > 0.0:
        u = torch.rand(shape, generator=g, device=device, dtype=torch.float32)
        x = torch.where(u < outlier_p, x * outlier_mul, x)
    return x.to(dtype)


def default_scale(head_dim):
    return 1.0 / math.sqrt(head_dim)
