"""Run a workload through the HIP library and the CPU oracle side by side.

Both sides receive the same seeded inputs; the oracle reads the very bytes
of the pinned host pool the GPU gathers from.  After every step the slot
table, hit mask, miss counts, miss list (id and victim slot per rank), the
state (Q, C, F) and the counters must be identical; the device slot buffer
is compared byte for byte at the checkpoints requested.
"""
from __future__ import annotations

import sys

import numpy as np

from oracle import Oracle


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def make_cfg(r, w, flags=0, gather_blocks=0, stage1_threads=0):
    return r.avsg_config_default(w.B, w.Nq, w.K, w.S, w.row_bytes, L=w.L, R=w.R,
                                 a1=w.a1, a2=w.a2, a_fp=w.afp, flags=flags,
                                 gather_blocks=gather_blocks,
                                 stage1_threads=stage1_threads)


class Pair:
    """A GPU handle and an oracle on one workload."""

    def __init__(self, w, gather=True, gather_blocks=0, shadow=True, stage1_threads=0,
                 flags=0, map_len=None):
        import torch
        import recall_step_amd as r
        self.r, self.torch, self.w = r, torch, w
        self.gather = gather
        self.no_reuse = bool(flags & r.FLAG_NO_REUSE)
        self.sort_merge = bool(flags & r.FLAG_SORT_MERGE)
        self.dense = bool(flags & r.FLAG_DENSE_MAP)
        # Dense matcher: one map entry per host row of the longest request
        # unless a shorter map is asked for.
        self.map_len = int(w.host_rows.max()) if map_len is None else int(map_len)
        self.host = r.HostPool(w.host_bytes) if gather else None
        if gather:
            w.fill_host_kv(self.host.array)
        flags |= 0 if gather else r.FLAG_SKIP_GATHER
        self.rs = r.RecallStep(make_cfg(r, w, flags, gather_blocks, stage1_threads),
                               self.host, w.host_rows_total,
                               map_len=self.map_len if self.dense else 0)
        self.oracle = Oracle.for_workload(
            w, host_kv=self.host.array if gather else None, shadow=shadow and gather)
        dev = self.rs.Q.device
        self.topk = torch.from_numpy(np.ascontiguousarray(w.topk)).to(dev)
        self.ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len)).to(dev)
        self.row_base = torch.from_numpy(w.row_base.astype(np.int64)).to(dev)
        self.host_rows = torch.from_numpy(w.host_rows.astype(np.int32)).to(dev)

    def io(self, t, **kw):
        return self.rs.io(self.topk[t], self.ctx[t], self.row_base, self.host_rows, **kw)

    def gpu_step(self, t):
        self.rs.step(self.io(t))

    def oracle_step(self, t):
        w = self.w
        if self.dense:
            return self.oracle.step_dense(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows,
                                          self.map_len)
        step = (self.oracle.step_no_reuse if self.no_reuse else
                self.oracle.step_sort_merge if self.sort_merge else self.oracle.step)
        return step(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows)

    def compare(self, ref, ctx, check_kv=False):
        torch = self.torch
        torch.cuda.synchronize()
        rs, o = self.rs, self.oracle
        st = rs.slot_table.cpu().numpy()
        hm = rs.hit_mask.cpu().numpy()
        nm = rs.n_miss.cpu().numpy()
        mp = rs.miss_pairs.cpu().numpy()
        assert np.array_equal(nm, ref.n_miss), f"{ctx}: n_miss"
        assert np.array_equal(hm, ref.hit_mask), f"{ctx}: hit_mask"
        assert np.array_equal(st, ref.slot_table), f"{ctx}: slot_table"
        B, Nq = nm.shape
        for b in range(B):
            for g in range(Nq):
                n = int(nm[b, g])
                assert np.array_equal(mp[b, g, :n], ref.miss_pairs[b, g, :n]), \
                    f"{ctx}: miss list of request {b} token {g}"
        assert np.array_equal(rs.Q.cpu().numpy(), o.Q), f"{ctx}: Q"
        assert np.array_equal(rs.C.cpu().numpy(), o.C), f"{ctx}: C"
        assert np.array_equal(rs.F.cpu().numpy(), o.F), f"{ctx}: F"
        assert np.array_equal(rs.CNT.cpu().numpy(), o.CNT), f"{ctx}: CNT"
        if self.dense:
            assert np.array_equal(rs.map.cpu().numpy(), o.map), f"{ctx}: map"
        if check_kv:
            assert np.array_equal(rs.dev_kv.cpu().numpy(), o.shadow), f"{ctx}: slot buffer"

    def close(self):
        self.rs.close()
        if self.host is not None:
            self.host.close()


def run_parity(w, steps=None, kv_every=None, gather=True, gather_blocks=0, label=None,
               stage1_threads=0, flags=0, map_len=None):
    """Step both sides through w, comparing everything after every step;
    returns the oracle's counters, int64 [B][8]."""
    label = label or w.name
    steps = w.steps if steps is None else steps
    say(f"[parity] {label}: B={w.B} Nq={w.Nq} K={w.K} S={w.S} L={w.L} R={w.R} "
        f"row={w.row_bytes} host_rows={w.host_rows_total} steps={steps} gather={gather}")
    p = Pair(w, gather=gather, gather_blocks=gather_blocks, stage1_threads=stage1_threads,
             flags=flags, map_len=map_len)
    try:
        for t in range(steps):
            p.gpu_step(t)
            ref = p.oracle_step(t)
            last = t == steps - 1
            check_kv = gather and (last or (kv_every is not None and t % kv_every == 0))
            p.compare(ref, f"{label} step {t}", check_kv=check_kv)
        return p.oracle.CNT.astype(np.int64)
    finally:
        p.close()
