"""The allocation-free entry point against avsg_step (needs a GPU).

avsg_step_noalloc keeps the miss list in a static device array shared by
every call on a device.  Two inputs in a row, the second smaller (matching:
B = 8, K = 2048; then tiny: B = 1, K = 256), each over a few steps: every
output, the state, the counters and the slot buffer equal those of
avsg_step with its allocated workspace, bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

from workloads import make

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recall_step_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


def _compare(ref, got, what):
    import torch
    torch.cuda.synchronize()
    for name in ("slot_table", "hit_mask", "n_miss", "Q", "C", "F", "CNT", "dev_kv"):
        a, b = getattr(ref, name), getattr(got, name)
        assert torch.equal(a, b), f"{what}: {name} differs"


def test_noalloc_step_equals_avsg_step_on_two_inputs_in_a_row():
    import torch
    import recall_step_amd as r
    for name, steps in (("matching", 3), ("tiny", 3)):
        w = make(name, steps=steps)
        _say(f"[no-alloc] {name}: B={w.B} K={w.K} S={w.S} steps={steps}")
        host = r.HostPool(w.host_bytes)
        w.fill_host_kv(host.array)
        cfg = r.avsg_config_default(w.B, w.Nq, w.K, w.S, w.row_bytes, L=w.L, R=w.R,
                                    a1=w.a1, a2=w.a2, a_fp=w.afp)
        ref = r.RecallStep(cfg, host, w.host_rows_total)
        got = r.RecallStep(cfg, host, w.host_rows_total)
        try:
            dev = ref.Q.device
            row_base = torch.from_numpy(w.row_base).to(dev)
            host_rows = torch.from_numpy(w.host_rows).to(dev)
            stream = torch.cuda.current_stream().cuda_stream
            torch.cuda.synchronize()
            for t in range(w.steps):
                topk = torch.from_numpy(np.ascontiguousarray(w.topk[t])).to(dev)
                ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len[t])).to(dev)
                # Neither call is given a miss list: avsg_step uses its
                # workspace, avsg_step_noalloc its static scratch.
                r.avsg_step(ref.handle, ref.io(topk, ctx, row_base, host_rows,
                                               miss_pairs=False), stream)
                r.avsg_step_noalloc(got.cfg, got.bufs,
                                    got.io(topk, ctx, row_base, host_rows, miss_pairs=False),
                                    stream)
                _compare(ref, got, f"{name} step {t}")
            assert int(got.CNT[:, r.CNT_MISSES].sum()) > 0
        finally:
            ref.close()
            got.close()
            host.close()
