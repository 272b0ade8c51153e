"""The gather probe (a measurement aid beside the attention path) reads exactly
the runs it is given: every workgroup's XOR of the 32-bit words it read
matches the XOR of the same words taken on the host, for the balanced split
of runs over workgroups the probe documents."""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_runs,run_bytes,workgroups", [(0, 16384, 3), (1, 16, 5), (37, 4096, 8),
                                                         (300, 16384, 41), (129, 1040, 64)])
def test_probe_reads_exactly_the_runs(gpu_lib, n_runs, run_bytes, workgroups):
    pk = gpu_lib
    print(f"probe n_runs={n_runs} run_bytes={run_bytes} workgroups={workgroups}", flush=True)
    rng = np.random.default_rng(n_runs * 7 + workgroups)
    kbuf = rng.integers(0, 2 ** 32, size=(1 << 20) // 4, dtype=np.uint32)    # 1 MiB each
    vbuf = rng.integers(0, 2 ** 32, size=(1 << 20) // 4, dtype=np.uint32)
    slots = (kbuf.nbytes - run_bytes) // 16 + 1
    ko = rng.integers(0, slots, size=n_runs).astype(np.int64) * 16
    vo = rng.integers(0, slots, size=n_runs).astype(np.int64) * 16
    assert np.all(ko + run_bytes <= kbuf.nbytes) and np.all(vo + run_bytes <= vbuf.nbytes)
    dev = "cuda:0"
    dk = torch.from_numpy(kbuf.view(np.int32)).to(dev)
    dv = torch.from_numpy(vbuf.view(np.int32)).to(dev)
    sink = torch.full((workgroups,), -1, dtype=torch.int32, device=dev)
    pk.kv_probe_gather(dk.data_ptr(), dv.data_ptr(), torch.from_numpy(ko).to(dev),
                       torch.from_numpy(vo).to(dev), run_bytes, sink)
    got = sink.cpu().numpy().view(np.uint32)
    words = run_bytes // 4
    for c in range(workgroups):
        want = np.uint32(0)
        for u in range(c * n_runs // workgroups, (c + 1) * n_runs // workgroups):
            want ^= np.bitwise_xor.reduce(kbuf[ko[u] // 4: ko[u] // 4 + words])
            want ^= np.bitwise_xor.reduce(vbuf[vo[u] // 4: vo[u] // 4 + words])
        assert got[c] == want, (c, hex(got[c]), hex(want))
