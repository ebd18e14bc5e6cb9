"""Bit-exact parity of the HIP recall path with the CPU oracle (needs a GPU).

Every test calls the library through its C ABI (via the ctypes binding) and
compares against the oracle on the same seeded inputs: slot tables, hit
masks, miss counts, the miss list (eviction victims), the state tensors, the
counters and the device slot buffer, all bit for bit.
"""
from __future__ import annotations

import numpy as np
import pytest

from workloads import gen_fuzz, make

from _parity import Pair, run_parity, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import recall_step_amd  # noqa: F401  (fails loudly if the library is missing)
    yield


@pytest.mark.parametrize("chunk", range(4))
def test_fuzz_corpus(chunk):
    """Tiny random cases: padding, out-of-range and speculative ids, MTP,
    lost mappings, R in {0, 1, 3, S-1}, L in {1, 2, 3, 5}."""
    for seed in range(chunk, 160, 4):
        run_parity(gen_fuzz(seed), kv_every=1)


def test_tiny_full():
    cnt = run_parity(make("tiny"), kv_every=1).sum(0)
    assert cnt[1] == 16 * 256


def test_matching_full():
    run_parity(make("matching"), kv_every=16)


def test_mtp3_full():
    cnt = run_parity(make("mtp3"), kv_every=8)
    assert (cnt[:, 6] == 0).all()


def test_imbalanced_full():
    run_parity(make("imbalanced"), kv_every=16)


def test_residency_full():
    run_parity(make("residency"), kv_every=32)


def test_more_requests_than_cus_at_the_largest_state():
    """300 requests of the residency shape (S = 8192: 132.5 KiB of LDS, one
    workgroup per CU), more workgroups than the 256 CUs, so they run in two
    rounds.  24 steps, so that the slot buffers fill and victims need the
    extra decay.  Stage One only: the host pool of 300 such requests would
    not fit host memory."""
    cnt = run_parity(make("residency", steps=24, B=300), gather=False, label="residency B=300")
    assert cnt[:, 5].sum() > 0  # live evictions: the buffers did fill


@pytest.mark.parametrize("K,S,threads", [(4096, 8192, 0), (1000, 1024, 256), (256, 512, 0),
                                         (2048, 8192, 512), (256, 16384, 0)])
def test_more_requests_than_cus_every_form(K, S, threads):
    """300 requests, more than the 256 CUs, so each workgroup takes several.
    The next request is loaded ahead with two state words per array per
    thread (K = 4096: four ids per thread) or one (S = 1024 at 256 threads;
    S = 512 with one id per thread); past two words (S = 8192 at 512
    threads, S = 16384 at 256) it is staged from memory.  Half of each
    selection carries over, so hits, refreshes and evictions all occur."""
    prev = {}

    def draw(rng, t, b):
        if b in prev:
            keep = rng.choice(prev[b], K // 2, replace=False)
            fresh = np.setdiff1d(rng.choice(3 * K, 2 * K, replace=False), keep)[: K - keep.size]
            ids = np.concatenate([keep, fresh])
        else:
            ids = rng.choice(3 * K, K, replace=False)
        prev[b] = ids
        return rng.permutation(ids).astype(np.int32)

    w = _stage_one_only(f"B=300 K={K} S={S}", K, S, 6, 300, 4 * K, draw)
    cnt = run_parity(w, gather=False, stage1_threads=threads)
    assert cnt[:, 0].sum() > 0 and cnt[:, 2].sum() > 0  # hits and misses


def test_more_requests_than_cus_with_query_tokens():
    """MTP-3 requests, 300 of them: the last query token of one request loads
    the next request's first ids, and invalidation runs per request."""
    run_parity(make("mtp3", steps=4, B=300), gather=False, label="mtp3 B=300")


@pytest.mark.parametrize("K,S", [(256, 512), (1000, 1024), (2048, 2048), (3000, 4096),
                                 (4096, 8192), (1, 16), (64, 64), (1501, 2048),
                                 (2999, 4096), (4095, 8192), (256, 16384), (1023, 16384)])
def test_shape_sweep_stage_one(K, S):
    """Ragged and maximal K, several S: every IPT template, the scalar path
    for K not a multiple of the ids per thread, and every slot-per-thread
    split of the Stage-One kernel, without the copy."""
    w = make("matching", steps=4)
    rng = np.random.default_rng([K, S])
    topk = np.full((4, 2, 1, K), -1, np.int32)
    for t in range(4):
        for b in range(2):
            n = max(1, K - int(rng.integers(0, 5)))
            topk[t, b, 0, :n] = rng.choice(65536, n, replace=False)
    w.topk, w.B, w.K, w.S, w.steps = topk, 2, K, S, 4
    w.ctx_len = w.ctx_len[:4, :2]
    w.host_rows, w.row_base = w.host_rows[:2], w.row_base[:2]
    run_parity(w, gather=False, label=f"sweep K={K} S={S}")


def _stage_one_only(name, K, S, steps, B, host_rows, draw):
    """A Stage-One-only workload whose selections come from draw(rng, t, b)."""
    w = make("matching", steps=steps)
    rng = np.random.default_rng([K, S, steps, B])
    topk = np.full((steps, B, 1, K), -1, np.int32)
    for t in range(steps):
        for b in range(B):
            ids = draw(rng, t, b)
            topk[t, b, 0, :ids.size] = ids
    w.name, w.topk, w.B, w.K, w.S, w.steps = name, topk, B, K, S, steps
    w.ctx_len = np.full((steps, B), host_rows, np.int32)
    w.host_rows = np.full(B, host_rows, np.int32)
    w.row_base = np.arange(B, dtype=np.int64) * host_rows
    return w


def test_wide_id_span_takes_the_sorting_path():
    """Misses spread over ids up to 2^30 exceed the rank bitmap's 2^18-id
    window, so those tokens order their misses by sorting; every other step
    keeps half of the previous selection, so hits and evictions occur too."""
    prev = {}

    def draw(rng, t, b):
        K = 2048
        if t % 2 == 1 and b in prev:
            keep = rng.choice(prev[b], K // 2, replace=False)
            fresh = rng.choice(1 << 30, K, replace=False)
            fresh = np.setdiff1d(fresh, keep)[: K - keep.size]
            ids = np.concatenate([keep, rng.permutation(fresh)])
        elif t % 3 == 2:
            ids = rng.choice(1 << 17, K, replace=False)    # narrow span
        else:
            ids = rng.choice(1 << 30, K, replace=False)
        prev[b] = ids.astype(np.int32)
        return rng.permutation(ids).astype(np.int32)

    w = _stage_one_only("wide span", 2048, 4096, 8, 3, 1 << 30, draw)
    cnt = run_parity(w, gather=False).sum(0)
    assert cnt[0] > 0 and cnt[5] > 0


@pytest.mark.parametrize("K,S,threads,gather", [(333, 1024, 0, False), (1001, 2048, 0, True),
                                                (1001, 2048, 256, False),
                                                (2001, 4096, 256, False)])
def test_token_length_not_a_multiple_of_ids_per_thread(K, S, threads, gather):
    """K that the ids per thread (2, 4 or 8 here) do not divide: one thread
    owns positions on both sides of K, whose ids past K must read as padding,
    and the outputs go out with scalar stores.  Ids come from a universe of
    3K, so about a third repeat from step to step."""
    def draw(rng, t, b):
        return rng.choice(3 * K, K, replace=False).astype(np.int32)

    w = _stage_one_only(f"K={K} threads={threads}", K, S, 5, 3, 3 * K, draw)
    cnt = run_parity(w, gather=gather, stage1_threads=threads)
    assert cnt[:, 0].sum() > 0 and cnt[:, 1].sum() == 5 * 3 * K


def test_query_tokens_switch_between_sorting_and_the_rank_bitmap():
    """Three query tokens per step, each ordering its misses either with the
    rank bitmap (ids below 2^16) or by sorting (ids up to 2^30, or a missing
    id repeated), in a pattern that changes with step and request.  So a
    token often starts after one that left the shared LDS region full of
    sort keys, miss pairs or bitmap bits.  Each token also selects a quarter
    of the previous token's ids, which that token installed: hits within the
    step."""
    K, S, Nq, B, steps, hr = 512, 2048, 3, 3, 6, 1 << 30
    rng = np.random.default_rng([23, K, S, Nq])
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    for t in range(steps):
        for b in range(B):
            prev = None
            for g in range(Nq):
                mode = (t + b + g) % 3
                n_keep = 0 if prev is None else K // 4
                keep = (rng.choice(prev, n_keep, replace=False) if n_keep
                        else np.zeros(0, np.int64))
                hi = (1 << 30) if mode == 0 else (1 << 16)
                fresh = np.setdiff1d(rng.choice(hi, K + n_keep, replace=False), keep)
                fresh = rng.permutation(fresh)[: K - n_keep]
                if mode == 2:
                    fresh[-1] = fresh[0]  # one missing id twice
                ids = rng.permutation(np.concatenate([keep, fresh])).astype(np.int32)
                topk[t, b, g] = ids
                prev = np.unique(ids)
    w = make("matching", steps=steps)
    w.name, w.topk, w.B, w.Nq, w.K, w.S, w.steps = ("tokens switch order paths", topk, B, Nq,
                                                    K, S, steps)
    w.ctx_len = np.full((steps, B), hr, np.int32)
    w.host_rows = np.full(B, hr, np.int32)
    w.row_base = np.arange(B, dtype=np.int64) * hr
    cnt = run_parity(w, gather=False)
    assert (cnt[:, 6] & 2).all() and cnt[:, 0].sum() > 0


def test_repeated_missing_ids_take_the_sorting_path():
    """A token that misses the same id twice: both copies get slots in
    (id, position) order and the duplicate error bit is set."""
    def draw(rng, t, b):
        ids = rng.choice(50000, 700, replace=False)
        dup = rng.choice(ids, 20, replace=False)
        return rng.permutation(np.concatenate([ids, dup])).astype(np.int32)

    w = _stage_one_only("repeated ids", 720, 2048, 5, 2, 50000, draw)
    cnt = run_parity(w, gather=False)
    assert (cnt[:, 6] & 2).all()


@pytest.mark.parametrize("threads", [256, 512, 1024])
@pytest.mark.parametrize("name", ["matching", "mtp3"])
def test_stage_one_workgroup_size_does_not_change_results(name, threads):
    """Every Stage-One workgroup size (ids per thread 8 down to 1 at K =
    2048) gives the oracle's results."""
    w = make(name, steps=6) if name == "matching" else make(name, steps=6, B=4)
    run_parity(w, gather=False, stage1_threads=threads, label=f"{name} T={threads}")


@pytest.mark.parametrize("part", ["request", "topk"])
@pytest.mark.parametrize("name", ["matching", "mtp3", "imbalanced"])
def test_gather_partitions_copy_the_same_rows(name, part):
    """The request-level and equal-top-K partitions the page compares
    against move the same rows into the same slots as the per-row split."""
    import recall_step_amd as r
    flag = r.FLAG_GATHER_BY_REQUEST if part == "request" else r.FLAG_GATHER_BY_TOPK
    w = make(name, steps=5) if name == "matching" else make(name, steps=5, B=6)
    run_parity(w, kv_every=1, flags=flag, label=f"{name} by {part}")


@pytest.mark.parametrize("gblocks", [0, 3])
def test_gather_partitions_on_fuzz_corpus(gblocks):
    """Tiny random cases (padding, out-of-range and speculative ids, MTP)
    under both comparison partitions, with the default grid and a grid
    smaller than the batch."""
    import recall_step_amd as r
    for seed in range(0, 160, 8):
        for flag in (r.FLAG_GATHER_BY_REQUEST, r.FLAG_GATHER_BY_TOPK):
            run_parity(gen_fuzz(seed), kv_every=1, flags=flag, gather_blocks=gblocks)


@pytest.mark.parametrize("name", ["tiny", "matching", "mtp3"])
def test_no_reuse_mode_matches_oracle(name):
    """"KV Offload": every valid selected row copied to slot g*K + i each
    step, in position order."""
    import recall_step_amd as r
    w = make(name, steps=4) if name != "mtp3" else make(name, steps=4, B=4)
    run_parity(w, kv_every=1, flags=r.FLAG_NO_REUSE, label=f"{name} no reuse")


def test_no_reuse_mode_on_fuzz_corpus():
    import recall_step_amd as r
    for seed in range(0, 160, 4):
        run_parity(gen_fuzz(seed), kv_every=1, flags=r.FLAG_NO_REUSE)
        run_parity(gen_fuzz(seed), kv_every=1,
                   flags=r.FLAG_NO_REUSE | r.FLAG_GATHER_BY_TOPK)


def test_sort_merge_matcher_on_fuzz_corpus():
    """The sort-merge comparison matcher against its oracle on tiny random
    cases (padding, out-of-range and speculative ids, MTP)."""
    import recall_step_amd as r
    for seed in range(0, 160, 4):
        run_parity(gen_fuzz(seed), kv_every=1, flags=r.FLAG_SORT_MERGE)


@pytest.mark.parametrize("name", ["matching", "reuse75_b8", "mtp3", "tiny"])
def test_sort_merge_matcher_on_workloads(name):
    import recall_step_amd as r
    w = make(name, steps=6) if name != "mtp3" else make(name, steps=4, B=4)
    cnt = run_parity(w, kv_every=2, flags=r.FLAG_SORT_MERGE, label=f"{name} sort-merge").sum(0)
    assert cnt[0] > 0


def test_sort_merge_repeated_missing_ids():
    import recall_step_amd as r

    def draw(rng, t, b):
        ids = rng.choice(50000, 700, replace=False)
        dup = rng.choice(ids, 20, replace=False)
        return rng.permutation(np.concatenate([ids, dup])).astype(np.int32)

    w = _stage_one_only("repeated ids", 720, 2048, 5, 2, 50000, draw)
    cnt = run_parity(w, gather=False, flags=r.FLAG_SORT_MERGE)
    assert (cnt[:, 6] & 2).all()


def test_layers_batched_equals_per_layer_and_oracle():
    """Two layers of the matching workload, each with its own cache: one
    batched launch per stage over the (layer, request) pairs gives the same
    outputs, state and slot buffer as one handle per layer, and both equal
    the oracle."""
    import torch
    import recall_step_amd as r
    from workloads.synth import gen_matching, stack_layers
    say("[parity] 2 layers, batched vs per layer")
    ws = [gen_matching(steps=4, layer=l) for l in range(2)]
    st = stack_layers(ws)
    cnt = run_parity(st, kv_every=1, label="matching x2 stacked").sum(0)
    assert cnt[1] == 4 * 16 * 2048
    p = Pair(st)
    try:
        B = ws[0].B
        per = []
        for l in range(2):
            cfg = r.avsg_config_default(B, st.Nq, st.K, st.S, st.row_bytes)
            per.append(r.RecallStep(cfg, p.host, st.host_rows_total))
        for t in range(st.steps):
            p.gpu_step(t)
            for l in range(2):
                sl = slice(l * B, (l + 1) * B)
                per[l].step(per[l].io(p.topk[t][sl], p.ctx[t][sl], p.row_base[sl],
                                      p.host_rows[sl]))
            torch.cuda.synchronize()
            for name in ("slot_table", "hit_mask", "n_miss", "Q", "C", "F", "CNT", "dev_kv"):
                both = torch.cat([getattr(per[l], name) for l in range(2)])
                assert torch.equal(both, getattr(p.rs, name)), f"step {t}: {name}"
        for h in per:
            h.close()
    finally:
        p.close()


def test_state_beyond_lds_is_unsupported():
    """K = S = 8192 needs more than 160 KiB of LDS: create refuses it."""
    import recall_step_amd as r
    cfg = r.avsg_config_default(1, 1, 8192, 8192, 1280, flags=r.FLAG_SKIP_GATHER)
    assert r.avsg_validate_config(cfg) == 0
    with pytest.raises(r.AvsgError) as e:
        r.RecallStep(cfg, None, 1 << 20)
    assert e.value.code == r.AVSG_EUNSUPPORTED


def test_largest_token_count_with_gather():
    """B * N_q = 16384 tokens, the most the gather's prologue scans: tiny
    requests (K = 4, S = 16) so that every token has a few misses."""
    from workloads.synth import Workload
    B, Nq, K, S, hr, steps = 4096, 4, 4, 16, 64, 3
    rng = np.random.default_rng(4096)
    topk = np.empty((steps, B, Nq, K), np.int32)
    for t in range(steps):
        for b in range(B):
            for g in range(Nq):
                topk[t, b, g] = rng.choice(hr, K, replace=False)
    w = Workload("4096 x 4 tokens", B, Nq, K, S, 16, steps, 4096, topk,
                 np.full((steps, B), hr, np.int32), np.full(B, hr, np.int32),
                 np.arange(B, dtype=np.int64) * hr, L=2, R=3)
    cnt = run_parity(w, kv_every=1)
    assert cnt[:, 2].sum() > 0 and cnt[:, 0].sum() > 0


def test_edge_inputs_of_each_request():
    """Requests whose inputs sit at the edges the method leaves to the
    caller, side by side in one batch: rows leaving the pool, a negative row
    base, no host rows, a verified length of 0, below 0 and beyond the rows,
    and an all-padding token.  Ids outside a request's valid rows are
    padding with the error bit, and invalidation follows N as given."""
    from workloads.synth import Workload
    B, Nq, K, S, steps = 8, 2, 8, 32, 6
    rb = np.array([0, 64, 250, 64, 128, 192, -5, 240], np.int64)
    hr = np.array([64, 0, 16, 64, 64, 64, 16, 16], np.int32)  # pool: 256 rows
    n_of = [64, 10, 16, 0, -3, 1000, 8, 8]
    rng = np.random.default_rng(99)
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    ctx = np.zeros((steps, B), np.int32)
    for t in range(steps):
        for b in range(B):
            ctx[t, b] = n_of[b]
            for g in range(Nq):
                if b == 0 and g == 1 and t % 2:
                    continue  # an all-padding token
                n = min(K, max(int(hr[b]), 1))
                topk[t, b, g, :n] = rng.choice(max(int(hr[b]), 16), n, replace=False)
    w = Workload("edge inputs", B, Nq, K, S, 64, steps, 99, topk, ctx, hr, rb, L=2, R=3)
    assert w.host_rows_total == 256
    cnt = run_parity(w, kv_every=1)
    assert (cnt[[1, 2, 6], 6] & 1).all()           # no rows, off the pool, negative base
    assert (cnt[[1, 2, 6], 0] == 0).all() and (cnt[[1, 2, 6], 2] == 0).all()
    assert cnt[[0, 3, 4, 5, 7], 2].min() > 0


def test_mtp_capacity_edge():
    """N_q * K == S with L = 1: the extra decay reaches its bound every token."""
    w = make("mtp3", steps=4, B=2)
    w.L = 1
    run_parity(w, kv_every=1, label="mtp3 L=1")


def test_state_init_resets_selected_rows():
    import torch
    w = make("tiny")
    w2 = make("tiny")
    # two requests over the same ids
    w2.B = 2
    w2.topk = np.concatenate([w.topk, w.topk[:, :, :, ::-1]], axis=1)
    w2.ctx_len = np.concatenate([w.ctx_len, w.ctx_len], axis=1)
    w2.host_rows = np.concatenate([w.host_rows, w.host_rows])
    w2.row_base = np.array([0, 4096], np.int64)
    say("[parity] state_init row mask")
    p = Pair(w2)
    try:
        for t in range(6):
            if t == 3:
                mask = torch.tensor([0, 1], dtype=torch.int32, device=p.rs.Q.device)
                p.rs.state_init(mask)
                p.oracle.Q[1] = -1
                p.oracle.C[1] = -1
                p.oracle.F[1] = -1
                p.oracle.CNT[1] = 0
            p.gpu_step(t)
            p.compare(p.oracle_step(t), f"row reset step {t}", check_kv=True)
    finally:
        p.close()


def test_match_then_gather_entry_points_and_workspace_miss_list():
    """avsg_match + avsg_gather with the miss list left in the library's
    workspace give the same slot buffer as avsg_step."""
    w = make("tiny")
    say("[parity] match/gather split, workspace miss list")
    p = Pair(w)
    try:
        for t in range(w.steps):
            io = p.io(t, miss_pairs=False)
            p.rs.match(io)
            p.rs.gather(io)
            ref = p.oracle_step(t)
            p.torch.cuda.synchronize()
            assert np.array_equal(p.rs.slot_table.cpu().numpy(), ref.slot_table)
        assert np.array_equal(p.rs.dev_kv.cpu().numpy(), p.oracle.shadow)
    finally:
        p.close()


def test_hip_graph_capture_and_replay():
    """One step captured in a HIP graph replays to the same results as the
    oracle; inputs change between replays through fixed buffers."""
    import torch
    w = make("matching", steps=8)
    say("[parity] graph capture matching x8")
    p = Pair(w)
    try:
        dev = p.rs.Q.device
        topk_in = torch.empty_like(p.topk[0])
        ctx_in = torch.empty_like(p.ctx[0])
        io = p.rs.io(topk_in, ctx_in, p.row_base, p.host_rows)
        # warm the first step eagerly (not captured), then capture step 1
        topk_in.copy_(p.topk[0])
        ctx_in.copy_(p.ctx[0])
        p.rs.step(io)
        p.compare(p.oracle_step(0), "graph eager step 0")
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                p.rs.step(io, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        for t in range(1, w.steps):
            topk_in.copy_(p.topk[t])
            ctx_in.copy_(p.ctx[t])
            g.replay()
            torch.cuda.synchronize()
            p.compare(p.oracle_step(t), f"graph replay step {t}", check_kv=True)
    finally:
        p.close()


def test_dense_map_in_a_captured_graph():
    """The dense matcher's step (map reads, clears and atomic maxima) replays
    from a captured graph to the oracle's results, map included."""
    import torch
    import recall_step_amd as r
    w = make("residency", steps=6, B=4)
    say("[parity] graph capture residency B=4 dense")
    p = Pair(w, flags=r.FLAG_DENSE_MAP)
    try:
        dev = p.rs.Q.device
        topk_in = torch.empty_like(p.topk[0])
        ctx_in = torch.empty_like(p.ctx[0])
        io = p.rs.io(topk_in, ctx_in, p.row_base, p.host_rows)
        topk_in.copy_(p.topk[0])
        ctx_in.copy_(p.ctx[0])
        p.rs.step(io)
        p.compare(p.oracle_step(0), "dense graph eager step 0")
        s = torch.cuda.Stream(device=dev)
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(g, stream=s):
                p.rs.step(io, stream=s)
        torch.cuda.current_stream().wait_stream(s)
        for t in range(1, w.steps):
            topk_in.copy_(p.topk[t])
            ctx_in.copy_(p.ctx[t])
            g.replay()
            torch.cuda.synchronize()
            p.compare(p.oracle_step(t), f"dense graph replay step {t}", check_kv=True)
    finally:
        p.close()


def test_two_handles_on_two_streams_concurrently():
    """Two handles stepped on two streams at once, each against its own
    oracle: the library keeps no state between handles."""
    import torch
    say("[parity] two handles, two streams")
    pa = Pair(make("matching", steps=6))
    pb = Pair(make("residency", steps=6, B=4))
    try:
        sa = torch.cuda.Stream(device=pa.rs.Q.device)
        sb = torch.cuda.Stream(device=pb.rs.Q.device)
        sa.wait_stream(torch.cuda.current_stream())
        sb.wait_stream(torch.cuda.current_stream())
        for t in range(6):
            pa.rs.step(pa.io(t), stream=sa)
            pb.rs.step(pb.io(t), stream=sb)
            torch.cuda.synchronize()
            pa.compare(pa.oracle_step(t), f"stream A step {t}", check_kv=t == 5)
            pb.compare(pb.oracle_step(t), f"stream B step {t}", check_kv=t == 5)
    finally:
        pa.close()
        pb.close()


def test_determinism_repeat_from_same_state():
    import torch
    w = make("matching", steps=3)
    say("[parity] determinism")
    p = Pair(w, gather=False)
    try:
        p.gpu_step(0)
        p.gpu_step(1)
        snap = [x.clone() for x in (p.rs.Q, p.rs.C, p.rs.F, p.rs.CNT)]
        p.gpu_step(2)
        first = [x.clone() for x in (p.rs.Q, p.rs.C, p.rs.F, p.rs.CNT, p.rs.slot_table)]
        for dst, src in zip((p.rs.Q, p.rs.C, p.rs.F, p.rs.CNT), snap):
            dst.copy_(src)
        p.gpu_step(2)
        torch.cuda.synchronize()
        again = (p.rs.Q, p.rs.C, p.rs.F, p.rs.CNT, p.rs.slot_table)
        for a, b in zip(first, again):
            assert torch.equal(a, b)
    finally:
        p.close()


def test_prefetch_select_and_threshold_match_oracle():
    """Candidate selection and the moving-average threshold, bit for bit
    (float32 compare and float32 arithmetic on both sides), over thresholds
    of +-inf, caps of 0 / small / above K, and lengths beyond the row."""
    import torch
    import recall_step_amd as r
    from oracle import Oracle
    say("[parity] prefetch select / ema")
    rng = np.random.default_rng(11)
    B, K, row = 6, 512, 70000
    cfg = r.avsg_config_default(B, 1, K, 1024, 16, flags=r.FLAG_SKIP_GATHER)
    rs = r.RecallStep(cfg, None, 1 << 20)
    o = Oracle(B, 1, K, 1024, 15, 7, 1, 3, 5, 16, 1)
    dev = rs.Q.device
    try:
        for trial in range(6):
            sc = rng.standard_normal((B, row)).astype(np.float32)
            ctx = rng.integers(-5, row + 5000, B).astype(np.int32)
            theta = rng.normal(2.0, 0.5, B).astype(np.float32)
            theta[trial % B] = np.inf
            theta[(trial + 1) % B] = -np.inf
            cap = rng.choice([0, 7, 200, K, K + 100], B).astype(np.int32)
            t_sc = torch.from_numpy(sc).to(dev)
            t_ctx = torch.from_numpy(ctx).to(dev)
            t_th = torch.from_numpy(theta).to(dev)
            t_cap = torch.from_numpy(cap).to(dev)
            cand = torch.empty((B, K), dtype=torch.int32, device=dev)
            r.avsg_prefetch_select(rs.handle, t_sc.data_ptr(), row, t_ctx.data_ptr(),
                                   t_th.data_ptr(), t_cap.data_ptr(), cand.data_ptr(), 0)
            torch.cuda.synchronize()
            ref = o.prefetch_select(sc, ctx, theta, cap)
            assert np.array_equal(cand.cpu().numpy(), ref), f"trial {trial}"
            kth = rng.normal(1.0, 1.0, B).astype(np.float32)
            for alpha in (0.5, 0.3):
                r.avsg_ema_threshold(rs.handle, torch.from_numpy(kth).to(dev).data_ptr(),
                                     t_th.data_ptr(), alpha, 0)
                torch.cuda.synchronize()
                theta = Oracle.ema_threshold(kth, theta, alpha)
                assert np.array_equal(t_th.cpu().numpy(), theta)
    finally:
        rs.close()


def test_prefetch_then_exact_equals_two_token_step():
    """Prefetch candidates matched first, then the exact top-K as a
    continuation of the same step, equal the oracle's one step over the two
    tokens in that order: outputs of both calls, state, counters and slot
    buffer after every step; the threshold follows the oracle's average."""
    import torch
    import recall_step_amd as r
    from oracle import Oracle
    w = make("scored", steps=6, B=4)
    say("[parity] scored B=4: prefetch + continuation vs 2-token oracle step")
    host = r.HostPool(w.host_bytes)
    w.fill_host_kv(host.array)
    cfg = r.avsg_config_default(w.B, 1, w.K, w.S, w.row_bytes)
    rs = r.RecallStep(cfg, host, w.host_rows_total)
    o = Oracle(w.B, 2, w.K, w.S, w.L, w.R, w.a1, w.a2, w.afp, w.row_bytes,
               w.host_rows_total, host_kv=host.array)
    dev = rs.Q.device
    try:
        scores = torch.from_numpy(w.extra["scores"]).to(dev)
        kth = torch.from_numpy(w.extra["kth"]).to(dev)
        topk = torch.from_numpy(np.ascontiguousarray(w.topk)).to(dev)
        ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len)).to(dev)
        row_base = torch.from_numpy(w.row_base).to(dev)
        host_rows = torch.from_numpy(w.host_rows).to(dev)
        theta = torch.full((w.B,), float("inf"), dtype=torch.float32, device=dev)
        cap = torch.full((w.B,), w.K, dtype=torch.int32, device=dev)
        cand = torch.empty((w.B, 1, w.K), dtype=torch.int32, device=dev)
        out1 = [torch.empty_like(x) for x in (rs.slot_table, rs.hit_mask, rs.n_miss,
                                              rs.miss_pairs)]
        theta_ref = np.full(w.B, np.inf, np.float32)
        ncand = 0
        for t in range(w.steps):
            r.avsg_prefetch_select(rs.handle, scores[t].data_ptr(), scores.shape[2],
                                   ctx[t].data_ptr(), theta.data_ptr(), cap.data_ptr(),
                                   cand.data_ptr(), 0)
            io1 = r.AvsgStepIO(cand.data_ptr(), ctx[t].data_ptr(), row_base.data_ptr(),
                               host_rows.data_ptr(), out1[0].data_ptr(), out1[1].data_ptr(),
                               out1[2].data_ptr(), out1[3].data_ptr())
            rs.match(io1)
            rs.gather(io1)
            io2 = rs.io(topk[t], ctx[t], row_base, host_rows)
            rs.match_continue(io2)
            rs.gather(io2)
            r.avsg_ema_threshold(rs.handle, kth[t].data_ptr(), theta.data_ptr(), 0.5, 0)
            torch.cuda.synchronize()
            c = o.prefetch_select(w.extra["scores"][t], w.ctx_len[t], theta_ref,
                                  np.full(w.B, w.K, np.int32))
            assert np.array_equal(cand.cpu().numpy()[:, 0], c), f"step {t}: candidates"
            ncand += int((c >= 0).sum())
            both = np.stack([c, w.topk[t, :, 0]], axis=1)
            ref = o.step(both, w.ctx_len[t], w.row_base, w.host_rows)
            for g, outs in ((0, [x.cpu().numpy() for x in out1]),
                            (1, [x.cpu().numpy() for x in (rs.slot_table, rs.hit_mask,
                                                           rs.n_miss, rs.miss_pairs)])):
                assert np.array_equal(outs[0][:, 0], ref.slot_table[:, g]), f"{t}/{g} slots"
                assert np.array_equal(outs[1][:, 0], ref.hit_mask[:, g]), f"{t}/{g} mask"
                assert np.array_equal(outs[2][:, 0], ref.n_miss[:, g]), f"{t}/{g} n"
                for b in range(w.B):
                    n = int(ref.n_miss[b, g])
                    assert np.array_equal(outs[3][b, 0, :n], ref.miss_pairs[b, g, :n])
            for name in ("Q", "C", "F", "CNT"):
                assert np.array_equal(getattr(rs, name).cpu().numpy(), getattr(o, name)), name
            assert np.array_equal(rs.dev_kv.cpu().numpy(), o.shadow), f"step {t}: slot buffer"
            theta_ref = Oracle.ema_threshold(w.extra["kth"][t], theta_ref, 0.5)
            assert np.array_equal(theta.cpu().numpy(), theta_ref)
        assert ncand > 0
    finally:
        rs.close()
        host.close()


def test_continuation_past_the_step_capacity_is_rejected():
    """The capacity bound N_q*K <= S (AVSG App. B, slot preservation) holds
    for a step as a whole: a continuation that would bring the step's query
    tokens past S/K returns AVSG_EINVAL and enqueues nothing; a new
    avsg_match starts a new count."""
    import torch
    import recall_step_amd as r
    K, S = 64, 128
    rng = np.random.default_rng(5)
    say("[parity] continuation capacity: B=2 K=64 S=128")
    for Nq, continues_ok in ((1, 1), (2, 0)):
        cfg = r.avsg_config_default(2, Nq, K, S, 16, flags=r.FLAG_SKIP_GATHER)
        rs = r.RecallStep(cfg, None, 1000)
        try:
            dev = rs.Q.device
            topk = torch.from_numpy(np.stack([
                np.stack([rng.choice(1000, K, replace=False) for _ in range(Nq)])
                for _ in range(2)]).astype(np.int32)).to(dev)
            ctx = torch.full((2,), 1000, dtype=torch.int32, device=dev)
            row_base = torch.tensor([0, 0], dtype=torch.int64, device=dev)
            host_rows = torch.full((2,), 1000, dtype=torch.int32, device=dev)
            io = rs.io(topk, ctx, row_base, host_rows)
            for _ in range(2):
                rs.match(io)
                for _ in range(continues_ok):
                    rs.match_continue(io)
                torch.cuda.synchronize()
                before = [getattr(rs, n).clone() for n in ("Q", "C", "F", "CNT")]
                with pytest.raises(r.AvsgError) as e:
                    rs.match_continue(io)
                assert e.value.code == r.AVSG_EINVAL
                torch.cuda.synchronize()
                for n, b in zip(("Q", "C", "F", "CNT"), before):
                    assert torch.equal(getattr(rs, n), b), n
        finally:
            rs.close()


# --- dense id -> slot map matcher (ECHO page, GPU cache manager) -----------

def test_dense_map_on_fuzz_corpus():
    """The dense matcher against its oracle on tiny random cases (padding,
    out-of-range and speculative ids, MTP), with a map covering every host
    row and with one covering half of them (ids past it are out of range)."""
    import recall_step_amd as r
    for seed in range(0, 160, 4):
        w = gen_fuzz(seed)
        run_parity(w, kv_every=1, flags=r.FLAG_DENSE_MAP, label=f"fuzz {seed} dense")
        run_parity(gen_fuzz(seed), flags=r.FLAG_DENSE_MAP | r.FLAG_GATHER_BY_TOPK,
                   map_len=max(1, int(w.host_rows.max()) // 2), label=f"fuzz {seed} dense half")


@pytest.mark.parametrize("name", ["matching", "residency", "mtp3", "imbalanced"])
def test_dense_map_on_workloads(name):
    import recall_step_amd as r
    w = make(name, steps=6) if name != "mtp3" else make(name, steps=4, B=4)
    cnt = run_parity(w, kv_every=3, flags=r.FLAG_DENSE_MAP, label=f"{name} dense").sum(0)
    assert cnt[0] > 0 and cnt[3] == cnt[4] == 0


@pytest.mark.parametrize("threads", [256, 512])
def test_dense_map_workgroup_size_does_not_change_results(threads):
    import recall_step_amd as r
    run_parity(make("matching", steps=4), gather=False, stage1_threads=threads,
               flags=r.FLAG_DENSE_MAP, label=f"matching dense T={threads}")


def test_dense_map_repeated_missing_ids():
    """Repeated missing ids take the sorting path and several slots; the
    map keeps the largest of them."""
    import recall_step_amd as r

    def draw(rng, t, b):
        ids = rng.choice(50000, 700, replace=False)
        dup = rng.choice(ids, 20, replace=False)
        return rng.permutation(np.concatenate([ids, dup])).astype(np.int32)

    w = _stage_one_only("repeated ids dense", 720, 2048, 5, 2, 50000, draw)
    cnt = run_parity(w, gather=False, flags=r.FLAG_DENSE_MAP)
    assert (cnt[:, 6] & 2).all()


def test_dense_map_state_init_resets_map_rows():
    import torch
    import recall_step_amd as r
    w = make("residency", steps=6, B=3)
    say("[parity] dense state_init row mask")
    p = Pair(w, flags=r.FLAG_DENSE_MAP)
    try:
        for t in range(w.steps):
            if t == 3:
                mask = torch.tensor([1, 0, 1], dtype=torch.int32, device=p.rs.Q.device)
                p.rs.state_init(mask)
                for b in (0, 2):
                    p.oracle.C[b] = p.oracle.F[b] = p.oracle.Q[b] = -1
                    p.oracle.CNT[b] = 0
                    p.oracle.map[b] = -1
            p.gpu_step(t)
            p.compare(p.oracle_step(t), f"dense row reset step {t}", check_kv=True)
    finally:
        p.close()


def test_dense_map_continuation_equals_two_token_step():
    """avsg_match on tokens A then avsg_match_continue on tokens B equal the
    oracle's one dense step over (A, B) when no id reaches the verified
    length, map included."""
    import torch
    import recall_step_amd as r
    from oracle import Oracle
    w = make("residency", steps=6, B=4)
    assert (w.topk < w.ctx_len[:, :, None, None]).all()
    say("[parity] residency B=4 dense: match + continuation vs 2-token oracle step")
    map_len = int(w.host_rows.max())
    host = r.HostPool(w.host_bytes)
    w.fill_host_kv(host.array)
    cfg = r.avsg_config_default(w.B, 1, w.K, w.S, w.row_bytes, L=w.L, R=w.R, a1=w.a1,
                                a2=w.a2, a_fp=w.afp, flags=r.FLAG_DENSE_MAP)
    rs = r.RecallStep(cfg, host, w.host_rows_total, map_len=map_len)
    o = Oracle(w.B, 2, w.K, w.S, w.L, w.R, w.a1, w.a2, w.afp, w.row_bytes,
               w.host_rows_total, host_kv=host.array)
    dev = rs.Q.device
    try:
        topk = torch.from_numpy(np.ascontiguousarray(w.topk)).to(dev)
        ctx = torch.from_numpy(np.ascontiguousarray(w.ctx_len)).to(dev)
        row_base = torch.from_numpy(w.row_base).to(dev)
        host_rows = torch.from_numpy(w.host_rows).to(dev)
        for t in range(w.steps):
            u = (t + 3) % w.steps
            io1 = rs.io(topk[t], ctx[t], row_base, host_rows)
            rs.step(io1)
            torch.cuda.synchronize()
            first = [x.cpu().numpy() for x in (rs.slot_table, rs.hit_mask, rs.n_miss)]
            io2 = rs.io(topk[u], ctx[t], row_base, host_rows)
            rs.match_continue(io2)
            rs.gather(io2)
            torch.cuda.synchronize()
            second = [x.cpu().numpy() for x in (rs.slot_table, rs.hit_mask, rs.n_miss)]
            both = np.concatenate([w.topk[t], w.topk[u]], axis=1)
            ref = o.step_dense(both, w.ctx_len[t], w.row_base, w.host_rows, map_len)
            for g, outs in ((0, first), (1, second)):
                assert np.array_equal(outs[0][:, 0], ref.slot_table[:, g]), f"{t}/{g} slots"
                assert np.array_equal(outs[1][:, 0], ref.hit_mask[:, g]), f"{t}/{g} mask"
                assert np.array_equal(outs[2][:, 0], ref.n_miss[:, g]), f"{t}/{g} n"
            for name in ("C", "F", "CNT", "map"):
                assert np.array_equal(getattr(rs, name).cpu().numpy(), getattr(o, name)), name
            assert np.array_equal(rs.dev_kv.cpu().numpy(), o.shadow), f"step {t}: slot buffer"
    finally:
        rs.close()
        host.close()


@pytest.mark.parametrize("K,S", [(2048, 8192), (1000, 4096)])
def test_continuation_with_more_requests_than_cus(K, S):
    """300 requests, more than the CUs, so each workgroup takes several and
    loads the next one's state ahead, here without the once-per-step decay
    in the continuation: a match on token A then avsg_match_continue on
    token B equal the oracle's one step over (A, B), outputs of both calls,
    state and counters.  No id is at or beyond the verified length, so the
    invalidation at the end of the first call changes nothing."""
    import torch
    import recall_step_amd as r
    from oracle import Oracle
    B, hr, steps = 300, 4 * K, 4
    rng = np.random.default_rng([K, S, 300])
    toks = np.full((steps, B, 2, K), -1, np.int32)
    prev = [None] * B
    for t in range(steps):
        for b in range(B):
            for g in range(2):
                if prev[b] is not None:
                    keep = rng.choice(prev[b], K // 2, replace=False)
                    fresh = np.setdiff1d(rng.choice(hr, 2 * K, replace=False), keep)[: K - K // 2]
                    ids = np.concatenate([keep, fresh])
                else:
                    ids = rng.choice(hr, K, replace=False)
                prev[b] = ids
                toks[t, b, g] = rng.permutation(ids)
    say(f"[parity] continuation B=300 K={K} S={S}")
    cfg = r.avsg_config_default(B, 1, K, S, 16, flags=r.FLAG_SKIP_GATHER)
    rs = r.RecallStep(cfg, None, B * hr)
    o = Oracle(B, 2, K, S, cfg.L, cfg.R, cfg.a1, cfg.a2, cfg.a_fp, 16, B * hr, shadow=False)
    dev = rs.Q.device
    try:
        ctx = torch.full((B,), hr, dtype=torch.int32, device=dev)
        row_base = torch.arange(B, dtype=torch.int64, device=dev) * hr
        host_rows = torch.full((B,), hr, dtype=torch.int32, device=dev)
        out1 = [torch.empty_like(x) for x in (rs.slot_table, rs.hit_mask, rs.n_miss,
                                              rs.miss_pairs)]
        for t in range(steps):
            ta = torch.from_numpy(np.ascontiguousarray(toks[t, :, :1])).to(dev)
            tb = torch.from_numpy(np.ascontiguousarray(toks[t, :, 1:])).to(dev)
            io1 = r.AvsgStepIO(ta.data_ptr(), ctx.data_ptr(), row_base.data_ptr(),
                               host_rows.data_ptr(), out1[0].data_ptr(), out1[1].data_ptr(),
                               out1[2].data_ptr(), out1[3].data_ptr())
            rs.match(io1)
            rs.match_continue(rs.io(tb, ctx, row_base, host_rows))
            torch.cuda.synchronize()
            ref = o.step(toks[t], np.full(B, hr, np.int32), np.arange(B, dtype=np.int64) * hr,
                         np.full(B, hr, np.int32))
            for g, outs in ((0, [x.cpu().numpy() for x in out1]),
                            (1, [x.cpu().numpy() for x in (rs.slot_table, rs.hit_mask,
                                                           rs.n_miss, rs.miss_pairs)])):
                assert np.array_equal(outs[0][:, 0], ref.slot_table[:, g]), f"{t}/{g} slots"
                assert np.array_equal(outs[1][:, 0], ref.hit_mask[:, g]), f"{t}/{g} mask"
                assert np.array_equal(outs[2][:, 0], ref.n_miss[:, g]), f"{t}/{g} n"
                for b in range(B):
                    n = int(ref.n_miss[b, g])
                    assert np.array_equal(outs[3][b, 0, :n], ref.miss_pairs[b, g, :n]), \
                        f"{t}/{g} miss list of request {b}"
            for name in ("Q", "C", "F", "CNT"):
                assert np.array_equal(getattr(rs, name).cpu().numpy(), getattr(o, name)), name
        assert int(o.CNT[:, 0].sum()) > 0 and int(o.CNT[:, 2].sum()) > 0  # hits and misses
    finally:
        rs.close()


@pytest.mark.parametrize("chunk", range(4))
def test_random_medium_configs(chunk):
    """Random shapes across the supported range (K up to 4096, N_q up to 4,
    S up to 16384, B up to 300, several L and R, random hash multipliers),
    each with a random matcher (hash, dense map, sort-merge, no reuse) or
    copy partition, workgroup size and with or without the copy: every
    id-per-thread form, several requests per workgroup, padding,
    out-of-range and speculative ids, all against the oracle after every
    step."""
    import recall_step_amd as r
    from workloads import gen_medium
    for seed in range(chunk, 48, 4):
        w = gen_medium(seed)
        rng = np.random.default_rng([11, seed])
        # The largest S at most the drawn one whose state fits the LDS.
        while True:
            cfg = r.avsg_config_default(w.B, w.Nq, w.K, w.S, w.row_bytes, L=w.L, R=w.R)
            if r.avsg_stage1_lds_bytes(cfg) > 0 or w.S // 2 < w.Nq * w.K:
                break
            w.S //= 2
        w.R = min(w.R, w.S - 1)
        if r.avsg_stage1_lds_bytes(cfg) == 0:
            say(f"[parity] medium {seed}: K={w.K} S={w.S} does not fit the LDS; skipped")
            continue
        flags = int(rng.choice([0, 0, r.FLAG_DENSE_MAP, r.FLAG_GATHER_BY_REQUEST,
                                r.FLAG_GATHER_BY_TOPK, r.FLAG_SORT_MERGE, r.FLAG_NO_REUSE]))
        if flags == r.FLAG_SORT_MERGE and r.avsg_stage1_lds_bytes(r.avsg_config_default(
                w.B, w.Nq, w.K, w.S, w.row_bytes, flags=flags)) == 0:
            flags = 0  # the sort-merge matcher's keys do not fit the LDS at this S
        threads = int(rng.choice([0] + [t for t in (256, 512, 1024) if w.K <= 8 * t]))
        gather = bool(rng.random() < 0.75)
        run_parity(w, kv_every=1, gather=gather, flags=flags, stage1_threads=threads,
                   label=f"medium {seed} flags={flags} T={threads}")
