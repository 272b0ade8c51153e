"""Benchmark: paged decode attention on one MI355X.

Default workload (the one the metric is quoted on): one layer of a
Llama-3-8B-shaped decode batch -- h_q 32, h_kv 8, d_h 128, bf16, block size 16,
64 requests with contexts uniform on [512, 4096].  A step is one pass of the
whole hot path for one layer: one paged_attention_decode_append call writes
the new token's K and V and reads the whole cache (for bf16 one kernel does
both and merges its split pieces itself; --two-calls times kv_append +
paged_attention_decode instead).  Once per model step, i.e. every `layers`
steps, the host allocator also reserves blocks and maps the slot of every
request's new token, and the table/length/slot arrays go to the device; a
timed region shorter than `layers` steps that does not start a model step
(such as --steps 20 --warmup 5 with 32 layers) holds no reservation.  The pool
holds `layers` layers (32, as in Llama-3-8B) and the steps walk them in order,
so each step reads a layer whose K/V was last touched `layers - 1` steps
earlier, far beyond the 256 MB last-level cache, as in a real decode step.

Other workloads (--workload) are measured the same way: llama3_70b_long
(h_q 64, 4 requests of 32k-128k tokens), fp8 and int8 (8-bit caches, 128
requests of 1k-8k tokens with x8 outliers), llama3_8b_window (64 requests of
8k-16k tokens read through a 4096-token window plus 4 sink tokens, dead
pages released), prefix_churn (32 layers x 256 requests sharing a
2000-token prefix found in the prefix cache, 26 retired and admitted per
step; a step there is one model step over all 32 layers) and cow_fork
(copy-on-write page copies of 256 forks over 32 layers).

Prints one JSON line.  `value` is KV GB/s: K+V bytes of the valid tokens read
by the decodes of the timed steps over their wall time.
"""

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode-attention KV GB/s (% of HBM peak) + µs/step, Llama-3-8B shape"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0   # dense bf16 matrix peak of MI355X


def event_every(steps):
    """Per-call brackets (CallTimer(every=...)): every timed call up to 256
    steps, else every (steps // 256)-th."""
    return max(1, steps // 256)


class CallTimer:
    """HIP events on the launch stream around the timed calls.

    Runs of back-to-back calls (nothing else on the stream between them) are
    bracketed as a whole, two events per run, so no event sits between two
    calls: each event is a packet the command processor handles between
    kernels, a few microseconds per pair, which per-call brackets would add to
    every step.  A run's time per call is its elapsed time over its calls,
    launch gaps included.  `new_run(j)` is true for a step whose call follows
    other work on the stream (a host upload); it starts a new run.  With
    `every`, every `every`-th call is bracketed alone instead (for steps with
    another kernel before the timed call)."""

    def __init__(self, stream, steps, new_run=None, every=None):
        self.stream = stream
        self.begin = [None] * steps
        self.end = [None] * steps
        self.runs = []
        if every is not None:
            groups = [[j] for j in range(0, steps, every)]
        else:
            groups, j = [], 0
            while j < steps:
                k = j + 1
                while k < steps and not (new_run is not None and new_run(k)):
                    k += 1
                groups.append(list(range(j, k)))
                j = k
        for g in groups:
            b, e = TimingEvent(), TimingEvent()
            self.begin[g[0]] = b
            self.end[g[-1]] = e
            self.runs.append((b, e, g))

    def before(self, j):
        if self.begin[j] is not None:
            self.begin[j].record(self.stream)

    def after(self, j):
        if self.end[j] is not None:
            self.end[j].record(self.stream)

    def results(self, per_step_work):
        """(ms per call, work per call, calls) for every bracket."""
        ms = np.array([b.elapsed_ms(e) / len(g) for b, e, g in self.runs])
        work = np.array([float(np.mean([per_step_work[j] for j in g])) for _, _, g in self.runs])
        n = np.array([len(g) for _, _, g in self.runs])
        return ms, work, n


DEFAULT_LAYERS = {"llama3_8b": 32, "llama3_70b_long": 8, "fp8": 16, "int8": 16, "llama3_8b_window": 4}
DEFAULT_SEED = {"llama3_8b": 2, "llama3_70b_long": 3, "fp8": 5, "int8": 5, "prefix_churn": 4, "cow_fork": 6,
                "llama3_8b_window": 7, "prefill": 8, "ctx_sweep": 2}

# HBM bytes (read + written) per launch of the decode kernel in the default
# step of each workload, from the rocprofv3 FETCH_SIZE and WRITE_SIZE runs in
# profiles/decode_workloads_hbm_counters.md, scaled by the plain-copy
# calibration there (fetch x2, write x1).  They hold for the kernel source they
# were taken on, identified by its SHA-256; any other source reports null.
TRAFFIC_SOURCE = "paged_kv_cache_271_amd/csrc/decode.hip"
TRAFFIC_SHA256 = "82fdfc31accca2ee319bce921d179d13a66b41d228320e68c9f3950f6aa9dc1b"
TRAFFIC_BYTES = {"llama3_8b": 592_628_899, "fp8": 1_243_550_214, "llama3_70b_long": 1_348_120_755,
                 "int8": 1_238_546_374, "llama3_8b_window": 1_093_820_896}
# The same per launch of prefill_kernel and of block_copy_kernel, from
# profiles/prefill_llama3_8b_counters.md and
# profiles/block_copy_cow_fork_hbm_counters.md: (source, its SHA-256, bytes).
TRAFFIC_OTHER = {
    "prefill": ("paged_kv_cache_271_amd/csrc/prefill.hip",
                "c29ff9971de46489195d14c3f72811b7f02c516321dfdac52bb9772e2b1902a3", 407_242_084),
    "cow_fork": ("paged_kv_cache_271_amd/csrc/copy.hip",
                 "60ed0088c3233bc027dc247d46fa41f24757ec97b73b00f985caaa8e05e88fc7", 1_073_810_950),
}


def decode_kernel_name(dtype, head_dim, window, batch):
    """The decode kernel the library launches for such a step: the LDS-ring
    kernel for bf16, fp8 and int8 batches with head_dim 128 of up to 4096
    requests (windowed ones on bf16 caches), the register-streaming kernel
    otherwise."""
    ring = head_dim == 128 and batch <= 4096 and (dtype == "bf16" or (dtype in ("fp8", "int8") and not window))
    return "decode_ring_kernel" if ring else "decode_stream_kernel"


def measured_traffic(workload, two_calls_asked=False):
    import hashlib
    if two_calls_asked and workload in ("llama3_8b", "llama3_70b_long", "llama3_8b_window", "fp8", "int8"):
        return None  # their counters were taken on the fused kernel
    source, sha, table = TRAFFIC_SOURCE, TRAFFIC_SHA256, TRAFFIC_BYTES
    if workload in TRAFFIC_OTHER:
        source, sha, nbytes = TRAFFIC_OTHER[workload]
        table = {workload: nbytes}
    with open(os.path.join(ROOT, source), "rb") as f:
        if hashlib.sha256(f.read()).hexdigest() != sha:
            return None
    return table.get(workload)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1024)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", default="llama3_8b",
                    choices=["llama3_8b", "llama3_70b_long", "fp8", "int8", "prefix_churn", "cow_fork",
                             "llama3_8b_window", "prefill", "ctx_sweep"])
    ap.add_argument("--layers", type=int, default=0, help="layers in the pool (0: workload default)")
    ap.add_argument("--seed", type=int, default=-1, help="input seed (-1: workload default)")
    ap.add_argument("--partition", type=int, default=0,
                    help="tokens per piece (0: split the batch evenly over the decode waves)")
    ap.add_argument("--two-calls", action="store_true",
                    help="run the step as kv_append + paged_attention_decode instead of the "
                         "single paged_attention_decode_append call")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="run one plain 1 GiB device copy before timing (scales HBM byte counters)")
    a = ap.parse_args()
    if a.seed < 0:
        a.seed = DEFAULT_SEED[a.workload]
    return a


def log(msg):
    print(msg, file=sys.stderr, flush=True)


class TimingEvent:
    """A HIP event used only for timing.  Created with hipEventDisableSystemFence
    so that recording it does not write back and invalidate the caches (the
    default event's system-scope fence idles the GPU for several microseconds
    and would be charged to the step)."""
    _hip = None
    FLAGS = 0x20000000  # hipEventDisableSystemFence

    def __init__(self):
        import ctypes
        if TimingEvent._hip is None:
            TimingEvent._hip = ctypes.CDLL("libamdhip64.so")
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        err = TimingEvent._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), ctypes.c_uint(self.FLAGS))
        if err != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({err})")

    def record(self, stream):
        err = TimingEvent._hip.hipEventRecord(self.ev, self._ct.c_void_p(stream.cuda_stream))
        if err != 0:
            raise RuntimeError(f"hipEventRecord failed ({err})")

    def elapsed_ms(self, end):
        ms = self._ct.c_float()
        err = TimingEvent._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if err != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({err})")
        return ms.value

    def __del__(self):
        try:
            TimingEvent._hip.hipEventDestroy(self.ev)
        except Exception:
            pass


def copy_calibration(torch, dev):
    src = torch.empty(2 ** 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst
    log("copy calibration: 1 GiB read + 1 GiB written by one copy kernel")


def stream_copy_gbs(torch, dev, nbytes=2 ** 30, reps=5):
    """Bandwidth of a plain device-to-device copy of `nbytes` (read + written
    bytes over the mean time of `reps` copies): the box's practical HBM
    ceiling, reported beside the published peak."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    stream = torch.cuda.current_stream()
    e0, e1 = TimingEvent(), TimingEvent()
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_ms(e1) / reps
    del src, dst
    torch.cuda.empty_cache()
    return round(2 * nbytes / (ms * 1e-3) / 1e9, 1)


def decode_workload(args, torch, synth, pk, dev, spec=None, layers=0):
    """Single-layer decode steps over a multi-layer pool (see the module doc).
    `spec` / `layers` replace the workload's shape and pool depth (sweeps)."""
    name = args.workload
    w = spec or synth.WORKLOADS[name]
    dtype = w["dtype"]
    B, H, h_q, D = w["batch"], w["h_kv"], w["h_q"], w["head_dim"]
    L = layers or args.layers or DEFAULT_LAYERS[name]
    elem = 1 if dtype in ("fp8", "int8") else 2
    outlier = w.get("outlier_p", 0.0)
    total = args.warmup + args.steps
    model_steps = (total + L - 1) // L
    rng = synth.streams(args.seed)
    if "contexts" in w:
        ctx0 = np.array(w["contexts"], np.int32)
    else:
        ctx0 = synth.uniform_contexts(rng["contexts"], B, *w["ctx_range"]).astype(np.int32)
    final = ctx0 + model_steps          # every request grows by one token per model step
    MB = int((final.max() + 15) // 16)
    N = int(((final + 15) // 16).sum())
    order = synth.permutation(rng["free_order"], N)
    log(f"{name}: pool {L} layers x {N} blocks ({N * H * 16 * D * elem * 2 * L / 1e9:.1f} GB), "
        f"B={B}, ctx {ctx0.min()}..{ctx0.max()}, {model_steps} model steps")

    pool = pk.Pool(L, N, H, D, dtype, dev, initial_free_order=order)
    table = np.zeros((B, MB), np.int32)
    lens = np.zeros(B, np.int32)
    # prefill ctx0 - 1 tokens per request; each step appends one more
    slots0 = pool.batch_reserve(table, lens, ctx0 - 1)
    d_slots0 = torch.from_numpy(slots0).to(dev)
    T0 = len(slots0)
    in_dt = torch.bfloat16
    for layer in range(L):
        k = synth.device_normal((T0, H, D), 1000 + 2 * layer, dev, in_dt, outlier, 8.0)
        v = synth.device_normal((T0, H, D), 1001 + 2 * layer, dev, in_dt, outlier, 8.0)
        pool.append(layer, k, v, d_slots0)
        del k, v
    torch.cuda.synchronize()
    log("prefill done")
    sink, window = w.get("sink", 0), w.get("window", 0)
    if window:   # pages no windowed decode reads go back to the pool
        freed = pool.window_release(table, lens, sink, window)
        log(f"window {window} + {sink} sinks: {freed} pages released, {pool.num_free()} free")

    def read_tokens(n):
        n = n.astype(np.int64)
        return n if not window else np.minimum(n, np.minimum(n, sink) + window)

    # per (model step, layer) new-token K/V and queries, resident before timing
    k_new = synth.device_normal((model_steps, L, B, H, D), 7, dev, in_dt, outlier, 8.0)
    v_new = synth.device_normal((model_steps, L, B, H, D), 8, dev, in_dt, outlier, 8.0)
    q_all = synth.device_normal((model_steps, L, B, h_q, D), 9, dev, in_dt)
    out = torch.empty((B, h_q, D), dtype=in_dt, device=dev)
    ws = pool.new_workspace(B, h_q, int(final.max()), args.partition)   # counters zeroed once
    d_table = torch.empty((B, MB), dtype=torch.int32, device=dev)
    d_lens = torch.empty(B, dtype=torch.int32, device=dev)
    d_slots = torch.empty(B, dtype=torch.int32, device=dev)
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()
    state = {"max_ctx": 0, "kv": 0, "shadow": None}

    def host_reserve():
        slots = pool.batch_reserve(table, lens, np.ones(B, np.int32))
        if window:
            pool.window_release(table, lens, sink, window)
        # the first reservation sends the whole table; later ones send only
        # the entries that now name a block (at most one new page per
        # request; entries released to -1 are never read again and keep
        # their old block on the device)
        flat = table.reshape(-1)
        prev = state["shadow"]
        idx = (np.arange(B * MB) if prev is None else np.flatnonzero((flat != prev) & (flat >= 0)))
        state["shadow"] = flat.copy()
        n = len(idx)
        pinned = torch.empty(2 * n + 2 * B, dtype=torch.int32, pin_memory=True)
        pidx = torch.empty(n, dtype=torch.int64, pin_memory=True)
        pn = pinned.numpy()
        pn[:n] = flat[idx]
        pn[n:n + B] = lens
        pn[n + B:n + 2 * B] = slots
        pidx.numpy()[:] = idx
        dev_buf = pinned.to(dev, non_blocking=True)
        if n:
            d_table.view(-1).index_copy_(0, pidx.to(dev, non_blocking=True), dev_buf[:n])
        d_lens.copy_(dev_buf[n:n + B])
        d_slots.copy_(dev_buf[n + B:n + 2 * B])
        state["max_ctx"] = int(lens.max())
        state["kv"] = int(read_tokens(lens).sum()) * H * D * elem * 2

    # every pool type runs the fused step unless --two-calls (fp8 / int8: the
    # decode kernel re-quantises the new token's tile itself); windowed
    # 8-bit steps run the append kernel and the windowed decode in one call
    two_calls = args.two_calls

    def step(i, timer=None, j=0):
        s, r = divmod(i, L)
        if r == 0:
            host_reserve()
        if two_calls:
            pool.append(r, k_new[s, r], v_new[s, r], d_slots)
        if timer is not None:
            timer.before(j)
        if window and two_calls:
            pool.decode_window(r, q_all[s, r], d_table, d_lens, state["max_ctx"], scale, sink, window,
                               args.partition, out=out, workspace=ws)
        elif window:
            pool.decode_window_append(r, q_all[s, r], k_new[s, r], v_new[s, r], d_slots, d_table, d_lens,
                                      state["max_ctx"], scale, sink, window, args.partition, out=out,
                                      workspace=ws)
        elif two_calls:
            pool.decode(r, q_all[s, r], d_table, d_lens, state["max_ctx"], scale, args.partition,
                        out=out, workspace=ws)
        else:
            pool.decode_append(r, q_all[s, r], k_new[s, r], v_new[s, r], d_slots, d_table, d_lens,
                               state["max_ctx"], scale, args.partition, out=out, workspace=ws)
        if timer is not None:
            timer.after(j)
        return state["kv"]

    if args.copy_calibration:
        copy_calibration(torch, dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")

    # events bracket the timed calls: runs of fused calls between host
    # uploads, or (two calls per step) the decode call alone
    if two_calls:
        timer = CallTimer(stream, args.steps, every=event_every(args.steps))
    else:
        timer = CallTimer(stream, args.steps, new_run=lambda j: (args.warmup + j) % L == 0)
    per_step_kv = []
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for j in range(args.steps):
        per_step_kv.append(step(args.warmup + j, timer, j))
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the device table must name the host's block at every page a decode reads
    nb_now = (lens.astype(np.int64) + 15) // 16
    live = (table >= 0) & (np.arange(MB)[None, :] < nb_now[:, None])
    assert np.array_equal(d_table.cpu().numpy()[live], table[live]), "device block table out of date"
    dec_ms, dec_kv, dec_n = timer.results(per_step_kv)

    probe = None
    if spec is None and not window and (H % 4) == 0 and h_q // H <= 16:
        probe = gather_probe(pool, table, lens, L, H, D, elem, torch, pk, dev)
        log(f"gather probe: {probe['us']:.1f} us for {probe['bytes'] / 1e6:.1f} MB ({probe['gbs']:.0f} GB/s)")
    cpu = None
    if spec is None and not args.no_cpu_baseline:
        cpu = cpu_baseline(ctx0, T0, k_new, v_new, q_all, args, w, L, dev)
    config = {
        "workload": f"{name}_decode_layer",
        "cache_dtype": dtype, "batch": B, "h_q": h_q, "h_kv": H, "head_dim": D, "block_size": 16,
        "contexts": (list(w["contexts"]) if "contexts" in w else {"uniform": list(w["ctx_range"])}),
        "layers_in_pool": L, "partition_tokens": args.partition,
        **({"sink_tokens": sink, "window_tokens": window} if window else {}),
        "step": ("kv_append + " if two_calls else "") + ("paged_attention_decode_window" if window else
                                                         "paged_attention_decode")
                + ("" if two_calls else "_append"),
    }
    return dict(wall=wall, kv_total=float(sum(per_step_kv)), dec_ms=dec_ms, dec_kv=dec_kv, dec_n=dec_n,
                probe=probe,
                config=config, cpu=cpu, traffic=measured_traffic(name, args.two_calls), dtype={"fp8": "fp8-e4m3 K/V, bf16 q", "int8": "int8 K/V, bf16 q"}.get(dtype, "bf16"),
                kernel=("paged_attention_decode_window" if window else "paged_attention_decode")
                + ("" if two_calls else "_append") + f" call ({decode_kernel_name(dtype, D, window, B)}, merging "
                "its split pieces itself; a reduce kernel follows only for requests split into many pieces)",
                traffic_note=f"HBM bytes read + written per {decode_kernel_name(dtype, D, window, B)} launch "
                             "(rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated); null if the kernel source changed")


SWEEP_CTX = (512, 1024, 2048, 4096, 8192, 16384)


def ctx_sweep_workload(args, torch, synth, pk, dev):
    """The Llama-3-8B batch (64 requests) with one fixed context length per
    point, the fused step timed at each: the call time should be affine in the
    total context, t = a + bytes / R.  Reports R (the streaming rate) as the
    value, with the per-point times and the fixed cost a."""
    base = dict(synth.WORKLOADS["llama3_8b"])
    base.pop("ctx_range")
    B, H, D = base["batch"], base["h_kv"], base["head_dim"]
    pts = []
    last = None
    for c in SWEEP_CTX:
        spec = dict(base, contexts=tuple([c] * B))
        per_layer = B * c * H * D * 2 * 2
        layers = max(2, -(-4 * 10 ** 9 // per_layer))  # >= 4 GB of pool: every step reads cold lines
        r = decode_workload(args, torch, synth, pk, dev, spec=spec, layers=layers)
        call_us = float(np.average(r["dec_ms"], weights=r["dec_n"])) * 1e3
        kv = float(np.average(r["dec_kv"], weights=r["dec_n"]))
        pts.append((c, kv, call_us, r["wall"] / args.steps * 1e6))
        log(f"ctx {c}: {kv / 1e6:.1f} MB, call {call_us:.1f} us ({kv / call_us / 1e3:.0f} GB/s), "
            f"step {pts[-1][3]:.1f} us")
        last = r
        torch.cuda.empty_cache()
    x = np.array([p[1] for p in pts])
    y = np.array([p[2] for p in pts])
    slope, icept = np.polyfit(x, y, 1)          # us per byte, us
    fit = icept + slope * x
    r2 = 1.0 - float(((y - fit) ** 2).sum()) / float(((y - y.mean()) ** 2).sum())
    rate = 1.0 / slope / 1e3                     # GB/s
    log(f"affine fit: call = {icept:.1f} us + bytes / {rate:.0f} GB/s (R^2 {r2:.5f})")
    config = {"workload": "llama3_8b_ctx_sweep", "batch": B, "h_q": base["h_q"], "h_kv": H, "head_dim": D,
              "block_size": 16, "cache_dtype": "bf16", "step": "paged_attention_decode_append",
              "ctx_points": list(SWEEP_CTX),
              "kv_bytes": [int(p[1]) for p in pts],
              "us_per_call": [round(p[2], 2) for p in pts],
              "us_per_step_points": [round(p[3], 2) for p in pts],
              "fit_fixed_us": round(float(icept), 2), "fit_rate_gbs": round(rate, 1), "fit_r2": round(r2, 6)}
    return dict(wall=last["wall"], kv_total=last["kv_total"], dec_ms=last["dec_ms"], dec_kv=last["dec_kv"],
                dec_n=last["dec_n"], config=config, cpu=None, traffic=None, traffic_note="HBM counters not taken for this sweep",
                dtype="bf16", value=rate, metric="paged decode call: streaming rate of the affine fit "
                "over context length (GB/s), Llama-3-8B shape",
                kernel="paged_attention_decode_append call at the longest context (decode_ring_kernel + "
                       "piece merge)")


def churn_workload(args, torch, synth, pk, dev):
    """Model steps of the shared-prefix batch with churn: each step retires and
    admits 26 requests, then appends and decodes every one of the 32 layers."""
    import workloads
    w = synth.WORKLOADS["prefix_churn"]
    total = args.warmup + args.steps
    run = workloads.PrefixChurn(dev, layers=w["num_layers"], batch=w["batch"],
                                prefix=w["prefix_tokens"], suffix=w["suffix_range"], steps=total,
                                churn=w["churn"], seed=args.seed, reuse_inputs=True)
    log(f"prefix_churn: {run.N} blocks x {w['num_layers']} layers")
    for s in range(args.warmup):
        run.step(s)
    torch.cuda.synchronize()
    logical, unique = [], []
    run.admit_seconds = 0.0
    t0 = time.perf_counter()
    for s in range(args.steps):
        run.step(args.warmup + s)
        logical.append(run.logical_kv_bytes() * w["num_layers"])
        unique.append(run.unique_kv_bytes() * w["num_layers"])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    cpu = None if args.no_cpu_baseline else churn_cpu_baseline(run, args, torch, synth, dev)
    config = {"workload": "prefix_churn_model_step", "batch": w["batch"], "layers": w["num_layers"],
              "prefix_tokens": w["prefix_tokens"], "suffix_range": list(w["suffix_range"]),
              "churn_per_step": w["churn"], "partition_tokens": 0,
              "unique_kv_bytes_per_step": int(np.mean(unique)),
              "unique_kv_GBs": round(float(sum(unique)) / wall / 1e9, 1),
              "admission": "kv_prefix_match of the 2000-token prefix (125 pages)",
              "admission_host_us_per_request": round(run.admit_seconds / (args.steps * w["churn"]) * 1e6, 2)}
    return dict(wall=wall, kv_total=float(sum(logical)), dec_ms=None, dec_kv=None, config=config,
                cpu=cpu, dtype="bf16", kernel=None)


def cow_fork_workload(args, torch, synth, pk, dev):
    """Copy-on-write forks (parallel sampling / beam search): every step forks
    each of 256 parent requests (Llama-3-8B heads, 32 layers) whose only page
    is partly filled; the children reserve one token each through
    kv_batch_reserve_cow, one kv_block_copy call copies the 256 shared pages
    in every layer, and the children are retired again (host).  value = bytes
    the copy reads and writes per second of wall time."""
    B, L, H, D = 256, 32, 8, 128
    N = 2 * B + 8
    rng = synth.streams(args.seed)
    order = synth.permutation(rng["free_order"], N)
    pool = pk.Pool(L, N, H, D, "bf16", dev, initial_free_order=order)
    ptable = np.zeros((B, 1), np.int32)
    plen = np.zeros(B, np.int32)
    slots = pool.batch_reserve(ptable, plen, rng["contexts"].integers(1, 16, B).astype(np.int32))
    d_slots = torch.from_numpy(slots).to(dev)
    for layer in range(L):
        k = synth.device_normal((len(slots), H, D), 3000 + 2 * layer, dev, torch.bfloat16)
        v = synth.device_normal((len(slots), H, D), 3001 + 2 * layer, dev, torch.bfloat16)
        pool.append(layer, k, v, d_slots)
    page_bytes = H * 16 * D * 2
    moved = 2 * B * L * 2 * page_bytes          # read + written, K and V
    pinned = torch.empty(2 * B, dtype=torch.int32, pin_memory=True)
    d_pairs = torch.empty(2 * B, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    ones = np.ones(B, np.int32)

    def step(timer=None, j=0):
        ctable, clen = ptable.copy(), plen.copy()
        pool.retain_n(ctable.reshape(-1))           # the fork
        _, src, dst = pool.batch_reserve_cow(ctable, clen, ones)
        assert len(src) == B
        pn = pinned.numpy()
        pn[:B], pn[B:] = src, dst
        d_pairs.copy_(pinned, non_blocking=True)
        if timer is not None:
            timer.before(j)
        pool.block_copy(d_pairs[:B], d_pairs[B:])
        if timer is not None:
            timer.after(j)
        pool.release_n(ctable.reshape(-1))          # the children retire
        return moved

    if args.copy_calibration:
        copy_calibration(torch, dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # every copy follows its step's upload of the page pairs: bracketed alone
    timer = CallTimer(stream, args.steps, every=event_every(args.steps))
    t0 = time.perf_counter()
    total = 0
    for j in range(args.steps):
        total += step(timer, j)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms, dec_kv, dec_n = timer.results([moved] * args.steps)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cow_cpu_baseline(args, rng_seed=args.seed, B=B, L=L, H=H, D=D, N=N)
    config = {"workload": "cow_fork_page_copy", "forks_per_step": B, "layers": L, "h_kv": H, "head_dim": D,
              "cache_dtype": "bf16", "page_bytes_per_layer_kv": 2 * page_bytes,
              "bytes_moved_per_step": moved}
    return dict(wall=wall, kv_total=float(total), dec_ms=dec_ms, dec_kv=dec_kv, dec_n=dec_n,
                config=config, cpu=cpu, traffic=measured_traffic("cow_fork"),
                traffic_note="HBM bytes read + written per block_copy_kernel launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, "
                             "copy-calibrated); null if the kernel source changed", dtype="bf16",
                kernel="kv_block_copy call (block_copy_kernel), bytes read + written",
                metric="kv_block_copy GB/s (read + written), copy-on-write forks")


def prefill_workload(args, torch, synth, pk, dev):
    """Prompt processing: 8 Llama-3-8B-shaped requests (h_q 32, h_kv 8, d 128)
    of 2048 new tokens each, their K/V already in a 4-layer pool; a step is
    one paged_attention_prefill call for one layer (layers rotate).  value =
    attention FLOP per second (2 per multiply-add: 2 d for each score and 2 d
    for each weighted V row, causal keys only)."""
    B, P, L, H, D, h_q = 8, 2048, 4, 8, 128, 32
    rng = synth.streams(args.seed)
    N = B * P // 16
    pool = pk.Pool(L, N, H, D, "bf16", dev, initial_free_order=synth.permutation(rng["free_order"], N))
    table = np.zeros((B, P // 16), np.int32)
    lens = np.zeros(B, np.int32)
    slots = pool.batch_reserve(table, lens, np.full(B, P, np.int32))
    d_slots = torch.from_numpy(slots).to(dev)
    for layer in range(L):
        k = synth.device_normal((B * P, H, D), 4000 + 2 * layer, dev, torch.bfloat16)
        v = synth.device_normal((B * P, H, D), 4001 + 2 * layer, dev, torch.bfloat16)
        pool.append(layer, k, v, d_slots)
        del k, v
    q_all = synth.device_normal((L, B * P, h_q, D), 4100, dev, torch.bfloat16)
    out = torch.empty((B * P, h_q, D), dtype=torch.bfloat16, device=dev)
    d_table = torch.from_numpy(table).to(dev)
    d_lens = torch.from_numpy(lens).to(dev)
    d_qs = torch.from_numpy(np.arange(B + 1, dtype=np.int32) * P).to(dev)
    flops = B * (P * (P + 1) // 2) * h_q * 4 * D
    scale = 1.0 / math.sqrt(D)
    stream = torch.cuda.current_stream()

    def step(i, timer=None, j=0):
        if timer is not None:
            timer.before(j)
        pool.prefill(i % L, q_all[i % L], d_table, d_lens, d_qs, P, P, scale, out=out)
        if timer is not None:
            timer.after(j)

    if args.copy_calibration:
        copy_calibration(torch, dev)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # back-to-back prefill calls: one run
    timer = CallTimer(stream, args.steps)
    t0 = time.perf_counter()
    for j in range(args.steps):
        step(args.warmup + j, timer, j)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dec_ms, dec_kv, dec_n = timer.results([flops] * args.steps)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = prefill_cpu_baseline(args, torch, synth, dev, q_all[(args.warmup + args.steps - 1) % L],
                                   (args.warmup + args.steps - 1) % L, B, P, H, h_q, D)
    config = {"workload": "llama3_8b_prefill_layer", "batch": B, "new_tokens": P, "h_q": h_q, "h_kv": H,
              "head_dim": D, "cache_dtype": "bf16", "layers_in_pool": L, "flop_per_step": flops}
    return dict(wall=wall, kv_total=float(flops) * args.steps, dec_ms=dec_ms,
                dec_kv=dec_kv, dec_n=dec_n, config=config, cpu=cpu, traffic=measured_traffic("prefill"),
                traffic_note="HBM bytes read + written per prefill_kernel launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, "
                             "copy-calibrated); null if the kernel source changed", dtype="bf16",
                kernel="paged_attention_prefill call (prefill_kernel)",
                metric="paged prefill attention TFLOP/s (causal, bf16 MFMA)", unit="TFLOP/s",
                bound="mfma", peak=MFMA_BF16_PEAK_TFLOPS, scale=1e12)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the paged decode "
              "path shards by request or by KV head with no exchange, and only the one-GPU "
              "measurement is built.", flush=True)
        sys.exit(2)

    import torch
    import synth
    import paged_kv_cache_271_amd as pk

    pk.load_library()
    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    dev = "cuda:0"
    torch.cuda.set_device(0)

    if args.workload == "prefix_churn":
        r = churn_workload(args, torch, synth, pk, dev)
    elif args.workload == "cow_fork":
        r = cow_fork_workload(args, torch, synth, pk, dev)
    elif args.workload == "prefill":
        r = prefill_workload(args, torch, synth, pk, dev)
    elif args.workload == "ctx_sweep":
        r = ctx_sweep_workload(args, torch, synth, pk, dev)
    else:
        r = decode_workload(args, torch, synth, pk, dev)
    # the metric's unit: GB/s (bytes per 1e9 s^-1) unless the workload counts FLOP
    unit_scale = r.get("scale", 1e9)
    unit = r.get("unit", "GB/s")
    peak = r.get("peak", HBM_PEAK_GBS)
    value = r["value"] if "value" in r else r["kv_total"] / r["wall"] / unit_scale
    ms_per_step = r["wall"] / args.steps * 1e3
    mean_kv = r["kv_total"] / args.steps
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.1f} us/step, {value:.0f} {unit}")
    roofline = None
    if r["dec_ms"] is not None:
        w_n = r["dec_n"]
        dec_mean_s = float(np.average(r["dec_ms"], weights=w_n)) / 1e3
        dec_p50_s = float(np.median(r["dec_ms"])) / 1e3
        kv_call = float(np.average(r["dec_kv"], weights=w_n))
        achieved = kv_call / dec_mean_s / unit_scale
        achieved_p50 = kv_call / dec_p50_s / unit_scale
        log(f"timed call {dec_mean_s * 1e6:.1f} us mean over {int(w_n.sum())} calls in {len(w_n)} brackets "
            f"(bracket p10 {np.percentile(r['dec_ms'], 10) * 1e3:.1f}, "
            f"p90 {np.percentile(r['dec_ms'], 90) * 1e3:.1f}), {achieved:.0f} {unit}")
        roofline = {
            "bound": r.get("bound", "hbm"),
            "kernel": r["kernel"],
            "achieved": round(achieved, 1),
            "peak": peak,
            "unit": unit,
            "frac": round(achieved / peak, 4),
            "frac_median_bracket": round(achieved_p50 / peak, 4),
            "traffic": r.get("traffic"),
            "traffic_note": r.get("traffic_note", "HBM bytes read + written per launch of the dominant "
                                  "kernel (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-calibrated); null if "
                                  "the kernel source changed"),
            "stream_copy_gbs": stream_copy_gbs(torch, dev),
            "us_per_call": round(dec_mean_s * 1e6, 2),
            "us_per_call_p10_p50_p90_bracket": [round(float(np.percentile(r["dec_ms"], x)) * 1e3, 2)
                                                for x in (10, 50, 90)],
            "calls_timed": int(w_n.sum()),
            "brackets": int(len(w_n)),
            "bracket_note": "HIP events on the launch stream around runs of back-to-back calls (a run ends at a "
                            "host upload or, for two calls per step, each decode call alone); time per call = "
                            "run time / calls, launch gaps included",
        }
        if r.get("probe"):
            pr = r["probe"]
            roofline["gather_probe"] = {
                "us_per_launch": round(pr["us"], 2), "bytes": pr["bytes"], "gbs": round(pr["gbs"], 1),
                "call_over_probe_time": round(dec_mean_s * 1e6 / pr["us"], 4),
                "note": "kv_probe_gather over the 16 KiB K and V runs of the final step's tables, same split "
                        "and grid as the decode, no arithmetic: the gather alone on this GPU",
            }
    config = dict(r["config"])
    config["us_per_step"] = round(ms_per_step * 1e3, 2)
    if unit == "GB/s":
        # logical bytes count the shared prefix once per request that reads it
        # (mostly served from cache): the HBM fraction uses the unique bytes
        unique = config.get("unique_kv_GBs")
        config["hbm_fraction"] = round((unique if unique is not None else value) / HBM_PEAK_GBS, 4)
        if unique is not None:
            config["hbm_fraction_of"] = "unique K/V bytes"
        config["kv_bytes_per_step"] = int(mean_kv)
    res = {
        "metric": r.get("metric", METRIC),
        "value": round(value, 1),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": r["dtype"],
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": r["cpu"],
    }
    print(json.dumps(res), flush=True)


def cpu_baseline(ctx0, slots0_len, k_new, v_new, q_all, args, w, L, dev):
    """The oracle on the host cores, on a bounded sample of the same decode
    workload: every (B / 16)-th request of the last decoded layer, as many as
    fit in 131072 tokens (at least one), one request per task on a thread pool
    as wide as the cores this process may use (at most 16), BLAS limited to one
    thread per task, repeated until about `cpu_seconds` have passed.

    What is timed is the oracle's decode of each sampled request as it
    stands: for bf16 caches the fp64 attention over the request's contiguous
    K/V (through the window's positions for a windowed workload); for fp8 and
    int8 caches the oracle pool's gather, which decodes the codes and applies
    the tile scales, followed by the same attention.  The inputs are
    regenerated from the same seeded generators (never read back from the
    GPU pool); the 8-bit codes come from the oracle's own append of those
    inputs, in the same calls the GPU pool received (the prefill in one call,
    then one token per model step)."""
    import torch
    import oracle
    import synth

    dtype = w["dtype"]
    B, H, h_q, D = w["batch"], w["h_kv"], w["h_q"], w["head_dim"]
    sink, window = w.get("sink", 0), w.get("window", 0)
    outlier = w.get("outlier_p", 0.0)
    last = args.warmup + args.steps - 1
    s_last, layer = divmod(last, L)
    to_bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    k_pre = synth.device_normal((slots0_len, H, D), 1000 + 2 * layer, dev, torch.bfloat16, outlier, 8.0)
    v_pre = synth.device_normal((slots0_len, H, D), 1001 + 2 * layer, dev, torch.bfloat16, outlier, 8.0)
    starts = np.concatenate([[0], np.cumsum(ctx0.astype(np.int64) - 1)])
    q = oracle.bf16_bits_to_f64(to_bits(q_all[s_last, layer]))
    scale = 1.0 / math.sqrt(D)
    sample, tokens = [], 0
    for b in range(0, B, max(1, B // 16)):
        n = int(ctx0[b]) + s_last
        if sample and (len(sample) == 16 or tokens + n > 131072):
            break
        sample.append(b)
        tokens += n
    tasks, read = [], 0
    for b in sample:
        kb = to_bits(torch.cat([k_pre[starts[b]:starts[b + 1]], k_new[:s_last + 1, layer, b]]))
        vb = to_bits(torch.cat([v_pre[starts[b]:starts[b + 1]], v_new[:s_last + 1, layer, b]]))
        n, n0 = kb.shape[0], int(ctx0[b]) - 1
        read += n if not window else min(n, min(n, sink) + window)
        if dtype in ("fp8", "int8"):
            pool = oracle.RefPool(1, (n + 15) // 16, H, D, dtype=dtype)
            pool.append(0, kb[:n0], vb[:n0], np.arange(n0))
            for t in range(n0, n):
                pool.append(0, kb[t:t + 1], vb[t:t + 1], [t])
            table = np.arange((n + 15) // 16)
            tasks.append(lambda b=b, pool=pool, table=table, n=n:
                         oracle.attention_fp64(q[b], *pool.gather_f64(0, table, n), scale))
        else:
            K, V = oracle.bf16_bits_to_f64(kb), oracle.bf16_bits_to_f64(vb)
            if window:
                tasks.append(lambda b=b, K=K, V=V:
                             oracle.attention_window_fp64(q[b], K, V, scale, sink, window))
            else:
                tasks.append(lambda b=b, K=K, V=V: oracle.attention_fp64(q[b], K, V, scale))
    del k_pre, v_pre
    elem = 1 if dtype in ("fp8", "int8") else 2
    kv_bytes = read * H * D * 2 * elem
    reps, dt, workers = _time_tasks(tasks, args.cpu_seconds)
    what = {"fp8": "fp8 codes (oracle pool gather + fp64 attention)",
            "int8": "int8 codes (oracle pool gather + fp64 attention)"}.get(dtype, "bf16 K/V")
    if window:
        what += f" through a {window}-token window + {sink} sinks"
    return {
        "value": round(kv_bytes * reps / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"fp64 oracle decode of {len(sample)} of {B} requests of one layer "
                  f"({kv_bytes / 1e6:.0f} MB of {what}), {reps} repetitions in {dt:.1f} s, "
                  f"one request per task on {workers} threads, BLAS limited to 1 thread per task",
    }


def gather_probe(pool, table, lens, L, H, D, elem, torch, pk, dev, launches=64, warm=8):
    """Time kv_probe_gather over the K/V runs the decode reads for the current
    tables: for every request b, set of four kv heads s and block j the
    decode's unit (b, s, j) reads the four adjacent tiles of heads 4s..4s+3 in
    block table[b][j], one run in K and one in V.  Units go in the decode's
    order over the decode's 768 workgroups.  Launches rotate over the pool's
    layers, as the decode steps do, and each is bracketed by HIP events on the
    launch stream; the reported time is the median launch.  Bytes are the
    runs' bytes (whole blocks)."""
    tile = 16 * D * elem
    offs = []
    for b in range(len(lens)):
        nb = (int(lens[b]) + 15) // 16
        for s in range(H // 4):
            offs.extend((int(table[b, j]) * H + 4 * s) * tile for j in range(nb))
    offs = np.array(offs, np.int64)
    assert offs.size and offs.min() >= 0 and offs.max() + 4 * tile <= pool.k_cache[0].numel() * pool.k_cache.element_size()
    d_off = torch.from_numpy(offs).to(dev)
    sink = torch.empty(768, dtype=torch.int32, device=dev)
    layer_bytes = pool.k_cache[0].numel() * pool.k_cache.element_size()
    kb, vb = pool.k_cache.data_ptr(), pool.v_cache.data_ptr()
    stream = torch.cuda.current_stream()
    # every event exists before the first launch and lives until the end, so
    # no event is created or destroyed between a record and its launch
    events = [(TimingEvent(), TimingEvent()) for _ in range(warm + launches)]
    torch.cuda.synchronize()
    for i, ev in enumerate(events):
        layer = i % L
        ev[0].record(stream)
        pk.kv_probe_gather(kb + layer * layer_bytes, vb + layer * layer_bytes, d_off, d_off, 4 * tile, sink)
        ev[1].record(stream)
    torch.cuda.synchronize()
    t_us = np.array([a.elapsed_ms(b) for a, b in events[warm:]]) * 1e3
    us = float(np.median(t_us))
    nbytes = int(offs.size) * 2 * 4 * tile
    log(f"gather probe launches: median {us:.1f} us, min {t_us.min():.1f}, max {t_us.max():.1f} over {len(t_us)}")
    return {"us": us, "bytes": nbytes, "gbs": nbytes / us / 1e3}


def cow_cpu_baseline(args, rng_seed, B, L, H, D, N):
    """The oracle's fork step on the same shape: the oracle allocator (same
    seeded free order) gives 256 parents one partly filled page each, every
    child retains its parent's page and reserves one token through the
    oracle's copy-on-write reservation, and the oracle pool copies the 256
    pages in every layer (K and V, bf16).  The copies are timed: 16 tasks of
    16 pages on a thread pool as wide as the process's cores (at most 16),
    repeated for about `cpu_seconds`.  Value: bytes read + written per second,
    as the workload's."""
    import oracle
    from oracle.prefix_cache import reserve_cow
    import synth
    rng = synth.streams(rng_seed)
    order = synth.permutation(rng["free_order"], N)
    alloc = oracle.RefAllocator(N, order)
    ptable, plen = [[] for _ in range(B)], [0] * B
    reserve_cow(alloc, ptable, plen, rng["contexts"].integers(1, 16, B).astype(np.int32))
    ctable, clen = [list(r) for r in ptable], list(plen)
    for r in ctable:
        for blk in r:
            alloc.retain(blk)
    _, pairs = reserve_cow(alloc, ctable, clen, [1] * B)
    assert len(pairs) == B
    pool = oracle.RefPool(L, N, H, D, 16, "bf16")
    # fill the pool so that every page is real memory (untouched zero pages
    # would make the reads nearly free)
    pool.K.fill(0x3F80)
    pool.V.fill(0x3F80)
    chunks = [pairs[i:i + 16] for i in range(0, len(pairs), 16)]
    tasks = [lambda c=c: pool.copy_pages([s_ for s_, _ in c], [d_ for _, d_ in c]) for c in chunks]
    reps, dt, workers = _time_tasks(tasks, args.cpu_seconds)
    moved = 2 * B * L * 2 * H * 16 * D * 2
    return {
        "value": round(moved * reps / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"oracle page copies of one fork step ({B} pages x {L} layers, K and V, bf16, "
                  f"{moved / 1e9:.2f} GB read + written), pairs from the oracle's copy-on-write "
                  f"reservation; {reps} repetitions in {dt:.1f} s, 16 pages per task on {workers} threads",
    }


def _time_tasks(tasks, seconds):
    """Run every task once per repetition on a thread pool as wide as the
    cores this process may use (at most 16), BLAS limited to one thread per
    task, until about `seconds` have passed.  Returns (repetitions, seconds,
    threads)."""
    from concurrent.futures import ThreadPoolExecutor
    from threadpoolctl import threadpool_limits
    reps = 0
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with threadpool_limits(limits=1), ThreadPoolExecutor(max_workers=workers) as ex:
        t0 = time.perf_counter()
        while True:
            list(ex.map(lambda f: f(), tasks))
            reps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    return reps, dt, workers


def churn_cpu_baseline(run, args, torch, synth, dev):
    """The fp64 oracle decode of every 16th of the 256 requests of the last
    layer, with the lengths they have after the timed steps: the layer's
    shared 2000-token prefix, regenerated from its seed, followed by the
    request's suffix.  The suffix values are the leading rows of the seeded
    input buffer the steps append from (the same shape and distribution; the
    exact rows a request took depend on the order of admissions).  Value:
    logical K/V GB/s, as the workload's."""
    import oracle
    layer = run.layers - 1
    to_bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    pk_ = oracle.bf16_bits_to_f64(to_bits(synth.device_normal(
        (run.prefix_len, 8, 128), run._seed("prefix_k", layer), dev, torch.bfloat16)))
    pv_ = oracle.bf16_bits_to_f64(to_bits(synth.device_normal(
        (run.prefix_len, 8, 128), run._seed("prefix_v", layer), dev, torch.bfloat16)))
    q = oracle.bf16_bits_to_f64(to_bits(run.reuse[2]))
    scale = 1.0 / math.sqrt(128)
    tasks, tokens = [], 0
    for b in range(0, run.batch, 16):
        n = int(run.lens[b])
        ns = n - run.prefix_len
        K = np.concatenate([pk_, oracle.bf16_bits_to_f64(to_bits(run.reuse[0][:ns]))])
        V = np.concatenate([pv_, oracle.bf16_bits_to_f64(to_bits(run.reuse[1][:ns]))])
        tasks.append(lambda b=b, K=K, V=V: oracle.attention_fp64(q[b], K, V, scale))
        tokens += n
    kv_bytes = tokens * 8 * 128 * 2 * 2
    reps, dt, workers = _time_tasks(tasks, args.cpu_seconds)
    return {
        "value": round(kv_bytes * reps / dt / 1e9, 4),
        "unit": "GB/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"fp64 oracle decode of {len(tasks)} of {run.batch} requests of one layer "
                  f"({kv_bytes / 1e6:.0f} MB of bf16 K/V, {run.prefix_len}-token prefix + suffix each), {reps} "
                  f"repetitions in {dt:.1f} s, one request per task on {workers} threads, BLAS limited "
                  f"to 1 thread per task",
    }


def prefill_cpu_baseline(args, torch, synth, dev, q_layer, layer, B, P, H, h_q, D):
    """The fp64 oracle prefill of every 16th query of the first request of
    the last layer run: query i over positions 0..i (the oracle called on
    that one query and its causal keys).  Inputs regenerated from the same
    seeds.  Value: attention TFLOP/s counted as the workload's."""
    import oracle
    to_bits = lambda t: t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    # the layer's K/V as appended (all requests, drawn in one call), request 0's rows
    K = oracle.bf16_bits_to_f64(to_bits(synth.device_normal((B * P, H, D), 4000 + 2 * layer, dev,
                                                            torch.bfloat16)[:P]))
    V = oracle.bf16_bits_to_f64(to_bits(synth.device_normal((B * P, H, D), 4001 + 2 * layer, dev,
                                                            torch.bfloat16)[:P]))
    q = oracle.bf16_bits_to_f64(to_bits(q_layer[:P]))
    scale = 1.0 / math.sqrt(D)
    rows = list(range(15, P, 16))
    tasks = [lambda i=i: oracle.prefill_attention_fp64(q[i:i + 1], K[:i + 1], V[:i + 1], scale)
             for i in rows]
    flops = sum(i + 1 for i in rows) * h_q * 4 * D
    reps, dt, workers = _time_tasks(tasks, args.cpu_seconds)
    return {
        "value": round(flops * reps / dt / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"fp64 oracle prefill of {len(rows)} of the {P} queries of one request of one layer "
                  f"(every 16th, each over its causal keys; {flops / 1e9:.2f} GFLOP), {reps} repetitions "
                  f"in {dt:.1f} s, one query per task on {workers} threads, BLAS limited to 1 thread per task",
    }


if __name__ == "__main__":
    main()
