"""The seeded input generators draw what their recipes say (no GPU needed).

Each workload stands in for one of the pages' settings, so the statistics the
recipe promises are checked: distinct ids per token, the recency window,
adjacent-step reuse, MTP overlap and speculative positions, long-tailed
lengths, and reproducibility from the seed alone.
"""
from __future__ import annotations

import numpy as np
import pytest

from workloads import gen_fuzz, gen_medium, make


def adjacent_reuse(w, g=0):
    r = []
    for t in range(1, w.steps):
        for b in range(w.B):
            a = w.topk[t, b, g]
            p = w.topk[t - 1, b, g]
            a, p = a[a >= 0], p[p >= 0]
            r.append(np.intersect1d(a, p).size / a.size)
    return float(np.mean(r))


@pytest.mark.parametrize("name,kw", [("tiny", {}), ("matching", {"steps": 4}),
                                     ("residency", {"steps": 4, "B": 4}),
                                     ("mtp3", {"steps": 4, "B": 3}),
                                     ("imbalanced", {"steps": 4, "B": 5}),
                                     ("reuse25_b1", {"steps": 4}),
                                     ("reuse75_b8", {"steps": 4})])
def test_reproducible_and_well_formed(name, kw):
    w1, w2 = make(name, **kw), make(name, **kw)
    assert np.array_equal(w1.topk, w2.topk) and np.array_equal(w1.ctx_len, w2.ctx_len)
    assert w1.topk.shape == (w1.steps, w1.B, w1.Nq, w1.K)
    assert w1.Nq * w1.K <= w1.S
    for t in range(w1.steps):
        for b in range(w1.B):
            for g in range(w1.Nq):
                ids = w1.topk[t, b, g]
                ids = ids[ids >= 0]
                assert np.unique(ids).size == ids.size          # distinct per token
                assert (ids < w1.host_rows[b]).all()
    assert w1.row_base[0] == 0
    assert (np.diff(w1.row_base) == w1.host_rows[:-1]).all()  # packed host rows


def test_tiny_keeps_70_percent_and_is_sorted():
    # 179 of 256 kept; new ids avoid only the kept ones, so a dropped id may
    # be drawn again (about 77 * 77 / 4096 ids per step)
    w = make("tiny")
    assert 179 / 256 <= adjacent_reuse(w) <= 179 / 256 + 0.02
    assert all((np.diff(w.topk[t, 0, 0]) > 0).all() for t in range(w.steps))


def test_matching_always_selects_the_recency_window():
    w = make("matching", steps=3)
    for t in range(w.steps):
        for b in range(w.B):
            assert np.isin(np.arange(65536 - 256, 65536), w.topk[t, b, 0]).all()


def test_residency_drift_is_15_percent_of_the_non_window_ids():
    w = make("residency", steps=6, B=3)
    # window (256) always kept; 1485 of 1792 others kept; the 307 fresh Zipf
    # draws avoid only the kept ids, so hot dropped ids come back now and then
    assert (256 + 1485) / 2048 <= adjacent_reuse(w) <= 0.88


def test_mtp3_tokens_overlap_and_reach_past_the_verified_length():
    w = make("mtp3", steps=2, B=2)
    for b in range(w.B):
        x0 = set(w.topk[0, b, 0].tolist())
        for g in (1, 2, 3):
            xg = w.topk[0, b, g]
            assert 0.55 <= len(x0 & set(xg.tolist())) / w.K <= 0.75
            assert (xg >= w.ctx_len[0, b]).sum() == g     # speculative positions


def test_imbalanced_lengths_are_clipped_lognormal():
    w = make("imbalanced", steps=2)
    assert w.host_rows.min() >= 2048 and w.host_rows.max() <= 262144
    assert 8192 <= np.median(w.host_rows) <= 32768


@pytest.mark.parametrize("name,reuse", [("reuse25_b1", 0.25), ("reuse75_b8", 0.75)])
def test_fixed_reuse_workloads(name, reuse):
    assert adjacent_reuse(make(name)) == pytest.approx(reuse)


def test_fuzz_respects_the_capacity_bound():
    for seed in range(50):
        w = gen_fuzz(seed)
        assert w.Nq * w.K <= w.S and w.S in (16, 32, 64)


def test_skewed_reuse_spans_its_range_per_request():
    """Each request of the skewed-reuse batch keeps its own share of the
    previous step's ids, evenly spread from 40 % to 100 %."""
    w = make("skew40to100_b8", steps=3)
    got = sorted(np.intersect1d(w.topk[2, b, 0], w.topk[1, b, 0]).size / w.K
                 for b in range(w.B))
    assert np.allclose(got, np.round(np.linspace(0.4, 1.0, w.B) * w.K) / w.K)


def test_medium_cases_are_reproducible_and_within_bounds():
    """The random medium cases: a pure function of the seed, within the
    capacity bound and the supported sizes, distinct ids per token apart
    from padding, and ids of each token inside the request's rows except
    the planted out-of-range ones."""
    for seed in range(32):
        w, w2 = gen_medium(seed), gen_medium(seed)
        assert np.array_equal(w.topk, w2.topk) and np.array_equal(w.ctx_len, w2.ctx_len)
        assert 1 <= w.K <= 4096 and 1 <= w.Nq <= 4 and w.Nq * w.K <= min(w.S, 8192)
        assert w.S & (w.S - 1) == 0 and 16 <= w.S <= 16384 and 1 <= w.B <= 300
        assert w.topk.shape == (w.steps, w.B, w.Nq, w.K)
        for t in range(w.steps):
            for b in range(w.B):
                hr = int(w.host_rows[b])
                assert 1 <= w.ctx_len[t, b] <= hr
                for g in range(w.Nq):
                    row = w.topk[t, b, g]
                    ids = row[(row >= 0) & (row < hr)]
                    assert np.unique(ids).size == ids.size
                    planted = row[(row != -1) & ((row < 0) | (row >= hr))]
                    assert planted.size <= 1
