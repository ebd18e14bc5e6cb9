"""Pins for the CPU oracle: what the pages and mathematics fix, not the oracle.

Page: "AVSG: Accelerated Vectorized Sparse Gather for Efficient KV Cache
Offload in Sparse-Attention LLM Serving" (sections named per test), and
"PulseInfer: I/O-Centric Sparse KV Cache Offloading" (recall as a set
difference of the selected blocks and the GPU-resident blocks).
"""
from __future__ import annotations

import json
import os

import numpy as np
import pytest

import oracle
from oracle import Oracle, rates
from workloads import gen_fuzz, make

from _ref import BruteState, DictSim, as_np_state, brute_step

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _oracle(B=1, Nq=1, K=4, S=8, L=2, R=1, a1=1, a2=1, afp=1 << 17,
            row_bytes=16, host_rows_total=None, host_rows=100):
    return Oracle(B, Nq, K, S, L, R, a1, a2, afp, row_bytes,
                  host_rows_total if host_rows_total is not None else B * host_rows)


def _step(o, topk, ctx, host_rows=100):
    B = o.B
    return o.step(np.asarray(topk, np.int32).reshape(B, o.Nq, o.K),
                  np.full(B, ctx, np.int32) if np.isscalar(ctx) else ctx,
                  np.arange(B, dtype=np.int64) * host_rows,
                  np.full(B, host_rows, np.int32))


# ------------------------------------------------------------- hash layer --

@pytest.mark.parametrize("S", [16, 64, 512, 8192])
def test_probe_sequence_is_a_permutation_when_R_is_S_minus_1(S):
    """Odd stride mod a power of two visits every bucket once (section 3.3:
    strides are forced odd); so with R = S-1 no probe can miss a reusable
    bucket."""
    rng = np.random.default_rng(S)
    for _ in range(5):
        a1, a2 = (int(v) * 2 + 1 for v in rng.integers(0, 2**31, 2))
        o = Oracle(1, 1, 1, S, 3, S - 1, a1, a2, 12345, 16, 1 << 20)
        for x in rng.integers(0, 1 << 30, 8):
            seq = o.probe_buckets(int(x))
            assert sorted(seq) == list(range(S))


def test_probe_home_and_stride_match_exact_integer_arithmetic():
    """h = (a1 x) mod S and d = ((a2 x) mod S) | 1 (section 3.3), checked
    against unbounded-integer arithmetic for ids near 2^31 where the 32-bit
    products wrap."""
    S, R = 4096, 3
    a1, a2 = 0x9E3779B1, 0x85EBCA77
    o = Oracle(1, 1, 1, S, 3, R, a1, a2, 1, 16, 1 << 31)
    for x in [0, 1, 7, 4095, 4096, 123456789, 2**31 - 1, 2**31 - 4097]:
        h, d = (a1 * x) % S, ((a2 * x) % S) | 1
        assert o.probe_buckets(x) == [(h + t * d) % S for t in range(R + 1)]


def test_word_packs_fingerprint_and_slot():
    """One packed word holds a fingerprint and a destination slot (App. B,
    "Collision and probe-budget semantics")."""
    o = Oracle(1, 1, 1, 64, 3, 3, 1, 1, 0xC2B2AE3D, 16, 100)
    for x, s in [(0, 0), (5, 63), (2**31 - 1, 17), (99999, 1)]:
        w = o.word(x, s)
        assert w >= 0 and w & 0xFFFF == s
        assert w >> 16 == ((x * 0xC2B2AE3D) % 2**32) >> 17


# ------------------------------------------------------ hand-worked case --

def test_handworked_s8_example():
    """A four-step case worked by hand from the page's rules (derivations in
    the fixture): a lost collision, an exhausted probe, invalidation of ids
    beyond the verified length, and an extra decay with live evictions."""
    with open(os.path.join(GOLDEN, "handworked_s8.json")) as f:
        case = json.load(f)
    p = case["params"]
    o = Oracle(p["B"], p["Nq"], p["K"], p["S"], p["L"], p["R"], p["a1"],
               p["a2"], p["afp"], p["row_bytes"], case["host_rows"])
    for st in case["steps"]:
        out = _step(o, st["topk"], st["ctx_len"], case["host_rows"])
        assert out.slot_table.ravel().tolist() == st["slot_table"]
        assert out.hit_mask.ravel().tolist() == st["hit_mask"]
        assert int(out.n_miss[0, 0]) == st["n_miss"]
        n = st["n_miss"]
        assert out.miss_pairs[0, 0, :n].tolist() == st["miss_pairs"]
        assert o.Q[0].tolist() == st["Q"]
        assert o.C[0].tolist() == st["C"]
        assert o.F[0].tolist() == st["F"]
        assert o.CNT[0].tolist() == st["CNT"]


# ----------------------------------------------------------- closed forms --

def test_disjoint_full_selections_map_rank_to_slot():
    """K = S and every step selects S fresh ids: everything misses, the extra
    decay reaches L, and the r-th smallest id lands in slot r (section 3.3
    allocation; misses ascending, lowest dead slots first)."""
    S, L = 64, 3
    o = Oracle(1, 1, S, S, L, 7, 0x9E3779B1, 0x85EBCA77, 0xC2B2AE3D, 16, 1 << 20)
    rng = np.random.default_rng(1)
    pool = rng.permutation(1 << 20)
    for t in range(5):
        X = pool[t * S:(t + 1) * S].astype(np.int32)
        out = _step(o, X, 1 << 20, 1 << 20)
        rank = np.argsort(np.argsort(X))
        assert (out.hit_mask == 0).all()
        assert out.slot_table.ravel().tolist() == rank.tolist()
        assert o.C[0].tolist() == sorted(X.tolist())
        assert (o.F[0] == L).all()
        if t > 0:
            assert int(o.CNT[0, oracle.LIVE_EVICTIONS]) == t * S


def test_repeated_selection_hits_everything_after_first_step():
    """Ids with distinct residues mod S never share a home bucket, so nothing
    is lost; repeating one selection then hits every id in its slot
    (section 3.1 hit definition; section 3.5 refresh keeps them alive)."""
    S, K = 256, 96
    rng = np.random.default_rng(2)
    X = (rng.permutation(S)[:K] + S * rng.integers(0, 50, K)).astype(np.int32)
    o = Oracle(1, 1, K, S, 2, 3, 0x9E3779B1, 0x85EBCA77, 0xC2B2AE3D, 16, 50 * S)
    first = _step(o, X, 50 * S, 50 * S)
    assert (first.hit_mask == 0).all()
    assert int(o.CNT[0, oracle.LOST_COLLISION]) == 0
    for _ in range(6):
        out = _step(o, X, 50 * S, 50 * S)
        assert (out.hit_mask == 1).all()
        assert (out.slot_table == first.slot_table).all()
        assert int(out.n_miss.sum()) == 0


@pytest.mark.parametrize("Nq", [2, 4])
def test_mtp_identical_tokens_reuse_closed_form(Nq):
    """From an empty buffer, N_q tokens that select the same ids share one
    reservation: reuse = (N_q - 1) / N_q exactly (section 3.6 progressive
    reuse; 4 tokens give 3/4)."""
    S, K = 512, 128
    X = (np.arange(K) * 3).astype(np.int32)
    o = Oracle(1, Nq, K, S, 4, 7, 0x9E3779B1, 0x85EBCA77, 0xC2B2AE3D, 16, 4096)
    out = o.step(np.tile(X, (1, Nq, 1)), np.array([4096], np.int32),
                 np.zeros(1, np.int64), np.array([4096], np.int32))
    assert int(out.n_miss[0, 0]) == K and int(out.n_miss[0, 1:].sum()) == 0
    hits, lookups = int(o.CNT[0, oracle.HITS]), int(o.CNT[0, oracle.LOOKUPS])
    copies = int(out.n_miss.sum())
    assert rates.reuse_rate(copies, lookups) == pytest.approx((Nq - 1) / Nq, abs=0)
    assert rates.hit_rate(hits, lookups) == pytest.approx((Nq - 1) / Nq, abs=0)
    for g in range(1, Nq):
        assert (out.slot_table[0, g] == out.slot_table[0, 0]).all()


def test_speculative_ids_miss_on_the_next_step():
    """Ids at or beyond the verified length N are emptied at end of step, so
    reselecting them misses and copies again (App. B, Speculative
    Invalidation; section 3.6)."""
    S, K = 64, 8
    o = _oracle(K=K, S=S, L=5, R=7, a1=0x9E3779B1, a2=0x85EBCA77, afp=0xC2B2AE3D)
    X = np.array([1, 2, 3, 40, 41, 42, 43, 44], np.int32)
    _step(o, X, 40)
    assert set(o.C[0][o.C[0] >= 0].tolist()) == {1, 2, 3}
    out = _step(o, X, 40)
    assert out.hit_mask.ravel().tolist() == [1, 1, 1, 0, 0, 0, 0, 0]


def test_padding_and_out_of_range_ids():
    """-1 is padding (slot -1, mask -1); other out-of-range ids are padding too
    and raise the sticky error bit; nothing else changes."""
    o = _oracle(K=6, S=16, R=3)
    out = _step(o, [5, -1, -7, 100, 101, 6], 100)
    assert out.slot_table.ravel().tolist()[1:5] == [-1] * 4
    assert out.hit_mask.ravel().tolist() == [0, -1, -1, -1, -1, 0]
    assert int(o.CNT[0, oracle.ERRORS]) == oracle.ERR_OUT_OF_RANGE
    assert int(o.CNT[0, oracle.LOOKUPS]) == 2


def test_request_with_rows_outside_pool_is_all_padding():
    o = Oracle(2, 1, 3, 16, 2, 3, 1, 1, 1 << 17, 16, 150)
    out = o.step(np.array([[[1, 2, 3]], [[1, 2, 3]]], np.int32),
                 np.array([100, 100], np.int32), np.array([0, 100], np.int64),
                 np.array([100, 100], np.int32))
    assert (out.hit_mask[0] == 0).all() and (out.hit_mask[1] == -1).all()
    assert o.CNT[:, oracle.ERRORS].tolist() == [0, 1]


def test_duplicate_ids_flagged_and_kept_separate():
    o = _oracle(K=4, S=16, R=3)
    out = _step(o, [9, 9, 3, -1], 100)
    assert int(o.CNT[0, oracle.ERRORS]) & oracle.ERR_DUPLICATE
    s = out.slot_table.ravel().tolist()
    assert s[0] != s[1] and min(s[:3]) >= 0


def _run_matcher(o, kind, topk, ctx, row_base, host_rows, map_len=100):
    if kind == "hash":
        return o.step(topk, ctx, row_base, host_rows)
    if kind == "dense":
        return o.step_dense(topk, ctx, row_base, host_rows, map_len)
    if kind == "sort_merge":
        return o.step_sort_merge(topk, ctx, row_base, host_rows)
    return o.step_no_reuse(topk, ctx, row_base, host_rows)


@pytest.mark.parametrize("kind", ["hash", "dense", "sort_merge", "no_reuse"])
def test_edge_inputs_of_every_matcher(kind):
    """Edge inputs through each step function: a verified length N <= 0
    empties every slot at the end of the step (every id is >= 0 >= N; App. B,
    Speculative Invalidation), so the next step misses everything; a token of
    padding only looks nothing up; a request with no host rows treats every
    id as out of range.  Request 0 is normal, 1 has N = 0, 2 has N = -5, 3
    selects only padding, 4 has no host rows."""
    B, Nq, K, S = 5, 2, 4, 16
    o = Oracle(B, Nq, K, S, 2, 3, 0x9E3779B1, 0x85EBCA77, 0xC2B2AE3D, 16, 500)
    # distinct residues mod S: distinct home buckets (a1 is odd), nothing lost
    X = np.tile(np.array([3, 8, 50, 69], np.int32), (B, Nq, 1))
    X[3] = -1
    ctx = np.array([100, 0, -5, 100, 100], np.int32)
    row_base = np.arange(B, dtype=np.int64) * 100
    host_rows = np.array([100, 100, 100, 100, 0], np.int32)
    for step in range(3):
        out = _run_matcher(o, kind, X, ctx, row_base, host_rows)
        assert (out.hit_mask[3] == -1).all() and (out.slot_table[3] == -1).all()
        assert (out.hit_mask[4] == -1).all() and (out.n_miss[3:] == 0).all()
        assert o.CNT[3, oracle.LOOKUPS] == 0 and o.CNT[4, oracle.LOOKUPS] == 0
        assert o.CNT[4, oracle.ERRORS] == oracle.ERR_OUT_OF_RANGE
        assert o.CNT[3, oracle.ERRORS] == 0
        for b in (0, 1, 2):
            assert o.CNT[b, oracle.LOOKUPS] == (step + 1) * Nq * K
        if kind == "no_reuse":
            continue
        for b in (1, 2):
            assert (o.C[b] == -1).all()
            # only the first token of each step copies: the later one hits
            # the rows the first one filled within the step
            assert out.n_miss[b].tolist() == [K, 0]
        if kind == "dense":
            assert (o.map[1:3] == -1).all()
        if step > 0:
            assert (out.hit_mask[0] == 1).all()
    assert (o.C[3] == -1).all() and (o.C[4] == -1).all()


def test_lifetime_survives_L_decays_then_dies():
    """A slot set to L stays reusable-protected for L unit decays and is
    reclaimable after L+1 (section 3.5; App. B slot preservation)."""
    L = 3
    o = _oracle(K=1, S=16, L=L, R=3)
    _step(o, [7], 100)
    slot = int(np.flatnonzero(o.C[0] == 7)[0])
    for k in range(1, L + 1):
        _step(o, [-1], 100)
        assert o.F[0, slot] == L - k
    _step(o, [-1], 100)
    assert o.F[0, slot] == -1


# -------------------------------------------------- brute force and sims --

def _fuzz_cases(n):
    return [gen_fuzz(s) for s in range(n)]


@pytest.mark.parametrize("chunk", range(4))
def test_oracle_matches_brute_force_transcription(chunk):
    """Every output and state entry agrees with the literal transcription on
    a fuzz corpus covering padding, out-of-range and speculative ids, MTP,
    R in {0, 1, 3, S-1} and L in {1, 2, 3, 5}."""
    for w in _fuzz_cases(400)[chunk::4]:
        o = Oracle.for_workload(w)
        st = BruteState(w.B, w.S)
        p = w.params()
        for t in range(w.steps):
            out = o.step(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows)
            O, H, n, pairs = brute_step(st, p, w.topk[t].tolist(), w.ctx_len[t].tolist(),
                                        w.row_base.tolist(), w.host_rows.tolist(),
                                        w.host_rows_total)
            Q, C, F, CNT = as_np_state(st)
            ctx = f"{w.name} step {t}"
            assert out.slot_table.tolist() == O, ctx
            assert out.hit_mask.tolist() == H, ctx
            assert out.n_miss.tolist() == n, ctx
            for b in range(w.B):
                for g in range(w.Nq):
                    assert out.miss_pairs[b, g, :n[b][g]].tolist() == [list(x) for x in pairs[b][g]], ctx
            assert (o.Q == Q).all() and (o.C == C).all() and (o.F == F).all(), ctx
            assert (o.CNT.astype(np.int64) == CNT).all(), ctx


def test_oracle_matches_dictionary_simulator_while_nothing_is_lost():
    """While no bucket mapping has been lost, the hash table is an exact
    dictionary of the cached ids, so the oracle must equal an LRU-with-aging
    simulator that has no hash table at all (section 3.5 aging; section 3.3
    allocation)."""
    compared = evictions = 0
    for seed in range(300):
        rng = np.random.default_rng([11, seed])
        S = int(rng.choice([32, 64]))
        Nq = int(rng.integers(1, 3))
        K = int(rng.integers(2, 9))
        L = int(rng.choice([1, 2, 3]))
        univ = int(rng.integers(2 * K, 4 * S))
        o = Oracle(1, Nq, K, S, L, S - 1, int(rng.integers(0, 2**31)) * 2 + 1,
                   int(rng.integers(0, 2**31)) * 2 + 1, 0xC2B2AE3D, 16, univ)
        sim = DictSim(S, L)
        for t in range(12):
            N = int(rng.integers(univ // 2, univ + 1))
            toks = [rng.choice(univ, K, replace=False).astype(np.int32) for _ in range(Nq)]
            before = o.CNT[0, oracle.LOST_COLLISION] + o.CNT[0, oracle.LOST_EXHAUSTED]
            out = o.step(np.array(toks)[None], np.array([N], np.int32),
                         np.zeros(1, np.int64), np.array([univ], np.int32))
            lost = o.CNT[0, oracle.LOST_COLLISION] + o.CNT[0, oracle.LOST_EXHAUSTED]
            res = sim.step([tk.tolist() for tk in toks], N)
            if before != 0 or (Nq > 1 and lost != 0):
                break
            # With one token, slots and hit flags are decided before the
            # step's link writes, so they agree even if the step loses a
            # mapping; with several tokens a loss can change later tokens.
            for g in range(Nq):
                for i, x in enumerate(toks[g].tolist()):
                    assert (int(out.slot_table[0, g, i]), int(out.hit_mask[0, g, i])) == res[g][x]
            assert o.C[0].tolist() == sim.C and o.F[0].tolist() == sim.F
            assert int(o.CNT[0, oracle.LIVE_EVICTIONS]) == sim.live_evictions
            compared += 1
            evictions = max(evictions, sim.live_evictions)
            if lost != 0:
                break
    assert compared > 1000 and evictions > 0


def test_hits_are_the_set_intersection_with_resident_ids():
    """Recall = selected \\ resident (PulseInfer page, recall stage): while
    nothing is lost, the hits of a single-token step are exactly the selected
    ids that the buffer caches before the step."""
    S, K = 1024, 24
    checked = 0
    for seed in range(40):
        rng = np.random.default_rng([5, seed])
        o = Oracle(1, 1, K, S, 4, S - 1, 0x9E3779B1, 0x85EBCA77, 0xC2B2AE3D, 16, 600)
        for t in range(40):
            resident = set(o.C[0][o.C[0] >= 0].tolist())
            X = rng.choice(600, K, replace=False).astype(np.int32)
            if int(o.CNT[0, 3] + o.CNT[0, 4]):
                break
            out = _step(o, X, 600, 600)
            hits = {int(x) for x, h in zip(X, out.hit_mask.ravel()) if h == 1}
            assert hits == set(X.tolist()) & resident
            assert {int(x) for x, h in zip(X, out.hit_mask.ravel()) if h == 0} == \
                set(X.tolist()) - resident
            checked += 1
    assert checked > 150


# ------------------------------------------------------------- invariants --

@pytest.mark.parametrize("name", ["tiny", "mtp3"])
def test_invariants_on_workloads(name):
    """After every step: every valid, non-speculative id's slot caches it
    (slots referenced earlier in a request survive the step, App. B slot
    preservation), slots are distinct within a token, lifetimes stay in
    [-1, L], hits + misses = valid lookups, and no hit has C[s] != x."""
    w = make(name) if name == "tiny" else make(name, steps=3, B=2)
    o = Oracle.for_workload(w)
    for t in range(w.steps):
        out = o.step(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows)
        for b in range(w.B):
            for g in range(w.Nq):
                X = w.topk[t, b, g]
                v = X >= 0
                s = out.slot_table[b, g][v]
                assert len(set(s.tolist())) == s.size
                keep = X[v] < w.ctx_len[t, b]
                assert (o.C[b][s[keep]] == X[v][keep]).all()
                assert (o.C[b][s[~keep]] == -1).all()
        assert o.F.min() >= -1 and o.F.max() <= w.L
        c = o.CNT.astype(np.int64)
        assert (c[:, oracle.HITS] + c[:, oracle.MISSES] == c[:, oracle.LOOKUPS]).all()


def test_probe_rounds_beyond_the_buckets_are_refused():
    """R + 1 > S rounds would only revisit buckets (odd stride modulo a
    power of two, section 3.3), so the oracle refuses R > S - 1 and accepts
    R = S - 1."""
    X = np.array([[[1, 2]]], np.int32)
    args = (np.array([100], np.int32), np.zeros(1, np.int64), np.array([100], np.int32))
    Oracle(1, 1, 2, 16, 2, 15, 1, 1, 1, 16, 100).step(X, *args)
    with pytest.raises(oracle.OracleError):
        Oracle(1, 1, 2, 16, 2, 16, 1, 1, 1, 16, 100).step(X, *args)


def test_capacity_bound_is_enforced():
    """N_q * K <= S is the capacity bound of App. B; the oracle refuses more."""
    o = Oracle(1, 2, 5, 8, 2, 1, 1, 1, 1, 16, 100)
    with pytest.raises(oracle.OracleError):
        o.step(np.zeros((1, 2, 5), np.int32), np.array([100], np.int32),
               np.zeros(1, np.int64), np.array([100], np.int32))


# ------------------------------------------------------------ data layer --

def test_gathered_rows_equal_host_rows_of_cached_ids():
    """After the copy, every slot a valid non-speculative id maps to holds that
    id's host row (section 3.4) -- true for any correct tie-breaking."""
    w = make("tiny")
    host = np.empty(w.host_bytes, np.uint8)
    w.fill_host_kv(host)
    o = Oracle.for_workload(w, host_kv=host)
    rows = host.reshape(-1, w.row_bytes)
    for t in range(w.steps):
        out = o.step(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows)
        X = w.topk[t, 0, 0]
        s = out.slot_table[0, 0]
        assert (o.shadow[0][s] == rows[w.row_base[0] + X]).all()


# ---------------------------------------------------------- printed rates --

def _golden_figures():
    rows = {}
    with open(os.path.join(GOLDEN, "paper_figures.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, inp, res, _ = [x.strip() for x in line.split("|")]
                kv = dict(tok.split("=") for tok in (inp + " " + res).split())
                rows[name] = {k: float(v) for k, v in kv.items()}
    return rows


def test_rate_definitions_reproduce_printed_figures():
    g = _golden_figures()
    m = g["mtp3_copies"]
    assert round(rates.copies_at_reuse(m["lookups"], m["reuse"])) == m["copies"]
    assert rates.reuse_rate(m["copies"], m["lookups"]) == pytest.approx(m["reuse"], abs=5e-5)
    gg = g["gain_8k"]
    assert round(rates.gain_pp(gg["hit_rate_pct"], gg["adjacent_pct"]), 2) == gg["gain_pp"]
    ml = g["matching_latency"]
    assert round(rates.latency_reduction(ml["before_us"], ml["after_us"]), 3) == ml["reduction"]
    tp = g["tpot"]
    # 1 - 55/91 = 39.6 %; the page prints the whole percent, 39 %.
    assert int(100 * rates.latency_reduction(tp["kv_offload_ms"], tp["avsg_ms"])) == \
        round(100 * tp["reduction"])
    assert rates.adjacent_reuse([1, 2, 3, 4], [3, 4, 5, 6]) == 0.5


# --- "KV Offload" comparison point (AVSG page, section 4.1) ---------------

@pytest.mark.parametrize("seed", range(40))
def test_no_reuse_copies_every_selected_row_every_step(seed):
    """With no reuse every valid selected id is transferred at every step
    (section 4.1): copies = valid ids, so the reuse rate 1 - copies / lookups
    of section 4.4 is 0; slots are distinct within a request, and after the
    copy each slot holds the host row of the id that maps to it."""
    w = gen_fuzz(seed)
    hk = np.random.default_rng([seed, 5]).integers(0, 256, w.host_bytes, dtype=np.uint8)
    o = Oracle.for_workload(w, host_kv=hk)
    for t in range(w.steps):
        before = o.CNT.astype(np.int64).copy()
        out = o.step_no_reuse(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows)
        d = (o.CNT.astype(np.int64) - before).sum(0)
        valid = 0
        for b in range(w.B):
            hr = int(w.host_rows[b])
            ok_rows = w.row_base[b] + hr <= w.host_rows_total
            slots = []
            for g in range(w.Nq):
                ids = w.topk[t, b, g]
                ok = (ids >= 0) & (ids < hr) & ok_rows
                valid += int(ok.sum())
                assert out.n_miss[b, g] == ok.sum()
                assert (out.hit_mask[b, g][ok] == 0).all()
                assert (out.hit_mask[b, g][~ok] == -1).all()
                assert (out.slot_table[b, g][~ok] == -1).all()
                slots += out.slot_table[b, g][ok].tolist()
                for i in np.flatnonzero(ok):
                    x, v = int(ids[i]), int(out.slot_table[b, g, i])
                    row = hk[(w.row_base[b] + x) * w.row_bytes:(w.row_base[b] + x + 1) * w.row_bytes]
                    assert np.array_equal(o.shadow[b, v], row)
            assert len(slots) == len(set(slots)) and all(0 <= v < w.S for v in slots)
        assert d[oracle.MISSES] == valid and d[oracle.LOOKUPS] == valid
        assert d[oracle.HITS] == 0


# --- sort-merge matcher comparison point (AVSG page, sections 2 and 4.2) ---

def _sort_merge_run(w, hk=None):
    o = Oracle.for_workload(w, host_kv=hk)
    outs, before = [], []
    for t in range(w.steps):
        before.append(o.C.copy())
        outs.append(o.step_sort_merge(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows))
    return o, outs, before


@pytest.mark.parametrize("seed", range(60))
def test_sort_merge_hits_are_the_set_intersection(seed):
    """Recall = selected minus resident (PulseInfer page, recall stage): for
    a single query token the hits are exactly the valid ids cached before the
    step, hits keep their row, the misses take increasing rows in increasing
    id order, and after the copy every slot holds its id's host row."""
    w = gen_fuzz(seed)
    w.Nq = 1
    w.topk = w.topk[:, :, :1, :].copy()
    hk = np.random.default_rng([seed, 7]).integers(0, 256, w.host_bytes, dtype=np.uint8)
    o, outs, before = _sort_merge_run(w, hk)
    for t, out in enumerate(outs):
        for b in range(w.B):
            hr = int(w.host_rows[b])
            ids = w.topk[t, b, 0]
            ok = (ids >= 0) & (ids < hr)
            cached = before[t][b]
            hit = ok & np.isin(ids, cached[cached >= 0])
            assert np.array_equal(out.hit_mask[b, 0] == 1, hit)
            assert np.array_equal(out.hit_mask[b, 0] == 0, ok & ~hit)
            for i in np.flatnonzero(hit):
                assert cached[out.slot_table[b, 0, i]] == ids[i]
            miss_i = np.flatnonzero(ok & ~hit)
            order = miss_i[np.lexsort((miss_i, ids[miss_i]))]
            assert (np.diff(out.slot_table[b, 0, order]) > 0).all()
            assert out.n_miss[b, 0] == miss_i.size
    t = w.steps - 1
    for b in range(w.B):
        ids = w.topk[t, b, 0]
        for i in np.flatnonzero(outs[t].hit_mask[b, 0] >= 0):
            x, v = int(ids[i]), int(outs[t].slot_table[b, 0, i])
            if x >= w.ctx_len[t, b]:
                continue
            lo = (w.row_base[b] + x) * w.row_bytes
            assert np.array_equal(o.shadow[b, v], hk[lo:lo + w.row_bytes])


def _sort_merge_oracle(case):
    p = case["params"]
    return Oracle(p["B"], p["Nq"], p["K"], p["S"], p["L"], p["R"], p["a1"], p["a2"],
                  p["afp"], p["row_bytes"], case["host_rows"])


def test_sort_merge_handworked_two_tokens():
    """Three steps of two query tokens worked by hand (derivations in the
    fixture): a later token's misses skip every row an earlier token of the
    same step hit or filled, an id cached in two rows hits the lower one, a
    row filled earlier in the step is a hit for a later token, and the rows
    of ids at or beyond N are emptied at the end of the step (AVSG page,
    sections 2, 3.6 and 4.2)."""
    with open(os.path.join(GOLDEN, "sort_merge_nq2_s8.json")) as f:
        case = json.load(f)
    o = _sort_merge_oracle(case)
    hr = case["host_rows"]
    for st in case["steps"]:
        out = o.step_sort_merge(np.asarray(st["topk"], np.int32).reshape(1, o.Nq, o.K),
                                np.array([st["ctx_len"]], np.int32),
                                np.zeros(1, np.int64), np.array([hr], np.int32))
        assert out.slot_table[0].tolist() == st["slot_table"]
        assert out.hit_mask[0].tolist() == st["hit_mask"]
        assert out.n_miss[0].tolist() == st["n_miss"]
        for g, n in enumerate(st["n_miss"]):
            assert out.miss_pairs[0, g, :n].tolist() == st["miss_pairs"][g]
        assert o.C[0].tolist() == st["C"]
        assert o.CNT[0].tolist() == st["CNT"]


@pytest.mark.parametrize("Nq", [2, 3, 4])
def test_sort_merge_identical_tokens_from_empty_reuse_closed_form(Nq):
    """N_q query tokens selecting the same K distinct ids from an empty
    buffer: the first token copies all K, every later token hits all K in
    the rows the first one filled, so reuse = (N_q - 1) / N_q exactly (the
    page's first-iteration reuse, section 4.4, for identical tokens)."""
    K, S = 32, 128
    rng = np.random.default_rng(Nq)
    X = rng.choice(5000, K, replace=False).astype(np.int32)
    o = Oracle(1, Nq, K, S, 3, 7, 1, 3, 5, 16, 5000)
    out = o.step_sort_merge(np.tile(X, (1, Nq, 1)), np.array([5000], np.int32),
                            np.zeros(1, np.int64), np.array([5000], np.int32))
    assert (out.hit_mask[0, 0] == 0).all()
    assert (out.hit_mask[0, 1:] == 1).all()
    for g in range(1, Nq):
        assert out.slot_table[0, g].tolist() == out.slot_table[0, 0].tolist()
    hits, lookups = int(o.CNT[0, oracle.HITS]), int(o.CNT[0, oracle.LOOKUPS])
    assert hits * Nq == (Nq - 1) * lookups


@pytest.mark.parametrize("seed", range(12))
def test_sort_merge_first_step_hits_are_overlaps_with_earlier_tokens(seed):
    """From an empty buffer, with N_q*K <= S, token g hits exactly the ids it
    shares with tokens 0..g-1 of the same step: every id an earlier token
    selected holds a row that no later token of the step may take (the page's
    progressive reuse across the tokens of one step, sections 3.6 and 4.4).
    Set arithmetic on the inputs, no buffer model."""
    rng = np.random.default_rng([seed, 11])
    Nq, K = int(rng.integers(2, 5)), int(rng.integers(4, 24))
    S = 1 << int(np.ceil(np.log2(Nq * K)))
    base = rng.choice(200, K, replace=False)
    X = np.empty((Nq, K), np.int32)
    for g in range(Nq):
        keep = rng.random(K) < 0.5
        fresh = rng.choice(np.setdiff1d(np.arange(400), base), K, replace=False)
        # distinct within the token; fresh draws of two tokens may coincide
        X[g] = np.where(keep, base, fresh)
        rng.shuffle(X[g])
    o = Oracle(1, Nq, K, S, 3, 7, 1, 3, 5, 16, 400)
    out = o.step_sort_merge(X.reshape(1, Nq, K), np.array([400], np.int32),
                            np.zeros(1, np.int64), np.array([400], np.int32))
    seen = set()
    for g in range(Nq):
        expect = np.isin(X[g], list(seen)) if seen else np.zeros(K, bool)
        assert np.array_equal(out.hit_mask[0, g] == 1, expect), g
        assert int(out.n_miss[0, g]) == int((~expect).sum())
        seen |= set(X[g].tolist())
    # every selected id of the step ends up cached, each in its own row
    cached = o.C[0][o.C[0] >= 0]
    assert sorted(cached.tolist()) == sorted(seen)


def test_sort_merge_with_s_equal_k_tracks_adjacent_step_reuse():
    """S = K and full, distinct selections: the buffer ends every step holding
    exactly that step's ids, so the hit rate of step t is the adjacent-step
    reuse |X_t & X_{t-1}| / K (section 4.4's definition) exactly."""
    w = make("reuse75_b8", steps=6)
    w.S = w.K
    o, outs, before = _sort_merge_run(w)
    for t in range(1, w.steps):
        for b in range(w.B):
            x = w.topk[t, b, 0]
            hits = int((outs[t].hit_mask[b, 0] == 1).sum())
            assert hits == np.intersect1d(x, w.topk[t - 1, b, 0]).size
            assert set(before[t][b].tolist()) == set(w.topk[t - 1, b, 0].tolist())


# --- threshold prefetch ahead of the recall (ECHO page, decode prefetch) ---

def _prefetch_oracle(B, K):
    return Oracle(B, 1, K, max(16, 1 << (2 * K - 1).bit_length()), 15, 7, 1, 3, 5, 16, 1)


def test_prefetch_extremes():
    """An infinite threshold prefetches nothing; minus infinity prefetches
    every position below N up to the cap, in order."""
    rng = np.random.default_rng(3)
    o = _prefetch_oracle(3, 64)
    sc = rng.standard_normal((3, 500)).astype(np.float32)
    ctx = np.array([500, 40, 300], np.int32)
    none = o.prefetch_select(sc, ctx, np.full(3, np.inf, np.float32), np.full(3, 64, np.int32))
    assert (none == -1).all()
    cap = np.array([64, 64, 10], np.int32)
    all_ = o.prefetch_select(sc, ctx, np.full(3, -np.inf, np.float32), cap)
    assert all_[0].tolist() == list(range(64))
    assert all_[1].tolist() == list(range(40)) + [-1] * 24
    assert all_[2].tolist() == list(range(10)) + [-1] * 54


@pytest.mark.parametrize("seed", range(5))
def test_prefetch_at_the_kplus1_score_is_the_exact_top_k(seed):
    """With the threshold at the (K+1)-th highest score and cap K, the
    candidates are exactly the top-K positions (numpy's partition), in
    ascending order: a perfect prediction prefetches the whole selection."""
    rng = np.random.default_rng(seed)
    K, n = 128, 4000
    o = _prefetch_oracle(2, K)
    sc = rng.standard_normal((2, n)).astype(np.float32)
    theta = np.array([np.partition(sc[b], n - K - 1)[n - K - 1] for b in range(2)], np.float32)
    cand = o.prefetch_select(sc, np.full(2, n, np.int32), theta, np.full(2, K, np.int32))
    for b in range(2):
        top = np.sort(np.argpartition(-sc[b], K - 1)[:K])
        assert np.array_equal(cand[b], top)


def test_prefetch_cap_keeps_the_first_positions():
    rng = np.random.default_rng(9)
    o = _prefetch_oracle(1, 256)
    sc = rng.standard_normal((1, 3000)).astype(np.float32)
    full = o.prefetch_select(sc, [3000], [0.5], [256])[0]
    capped = o.prefetch_select(sc, [3000], [0.5], [37])[0]
    assert np.array_equal(capped[:37], full[:37]) and (capped[37:] == -1).all()
    assert (np.diff(full[full >= 0]) > 0).all()


def test_ema_threshold_closes_the_gap_by_one_minus_alpha():
    """From +inf the first update takes the observed score; with a constant
    observed score s the gap theta - s shrinks by (1 - alpha) per step."""
    s = np.array([2.0, -1.5], np.float32)
    th = Oracle.ema_threshold(s, np.full(2, np.inf, np.float32), 0.5)
    assert np.array_equal(th, s)
    for alpha in (0.5, 0.25, 0.75, 1.0):
        th = np.array([10.0, 6.5], np.float32)
        for n in range(1, 12):
            th = Oracle.ema_threshold(s, th, alpha)
            assert np.allclose(th - s, (np.array([8.0, 8.0]) * (1 - alpha) ** n),
                               rtol=0, atol=1e-5), (alpha, n)


# --- dense id -> slot map (ECHO page, GPU cache manager) -------------------

def _dense_case(seed):
    rng = np.random.default_rng([21, seed])
    S = int(rng.choice([16, 32, 64]))
    Nq = int(rng.integers(1, 4))
    K = int(rng.integers(1, S // Nq + 1))
    L = int(rng.choice([1, 2, 3, 5]))
    univ = int(rng.integers(K, 4 * S + 1))
    return rng, S, Nq, K, L, univ


@pytest.mark.parametrize("chunk", range(6))
def test_dense_map_equals_dictionary_simulator(chunk):
    """The dense map is an exact dictionary, so with the same aging policy
    (AVSG page, sections 3.3 and 3.5) it must equal the dictionary simulator
    at every step, with several query tokens and with nothing ever lost:
    slots, hit flags, buffer state and counters."""
    steps = 0
    for seed in range(chunk * 50, chunk * 50 + 50):
        rng, S, Nq, K, L, univ = _dense_case(seed)
        o = Oracle(1, Nq, K, S, L, 1, 1, 1, 1, 16, univ)
        sim = DictSim(S, L)
        for t in range(10):
            N = int(rng.integers(univ // 2, univ + 1))
            toks = [rng.choice(univ, K, replace=False).astype(np.int32) for _ in range(Nq)]
            out = o.step_dense(np.array(toks)[None], np.array([N], np.int32),
                               np.zeros(1, np.int64), np.array([univ], np.int32), univ)
            res = sim.step([tk.tolist() for tk in toks], N)
            for g in range(Nq):
                for i, x in enumerate(toks[g].tolist()):
                    assert (int(out.slot_table[0, g, i]), int(out.hit_mask[0, g, i])) == res[g][x]
                assert out.n_miss[0, g] == sum(1 for v in res[g].values() if v[1] == 0)
            assert o.C[0].tolist() == sim.C and o.F[0].tolist() == sim.F
            assert int(o.CNT[0, oracle.LIVE_EVICTIONS]) == sim.live_evictions
            assert int(o.CNT[0, oracle.LOST_COLLISION]) == int(o.CNT[0, oracle.LOST_EXHAUSTED]) == 0
            mapped = {x: int(v) for x, v in enumerate(o.map[0].tolist()) if v >= 0}
            assert mapped == sim.slot_of
            steps += 1
    assert steps == 500


@pytest.mark.parametrize("seed", range(30))
def test_dense_map_equals_hash_matching_while_nothing_is_lost(seed):
    """Same allocation and aging (AVSG page, sections 3.3-3.5): while the
    hash table has lost no mapping it is an exact dictionary too, so both
    matchers give the same slots, flags, C, F and hit/miss counts."""
    w = gen_fuzz(seed)
    h = Oracle.for_workload(w)
    d = Oracle.for_workload(w)
    map_len = int(w.host_rows.max())
    for t in range(w.steps):
        oh = h.step(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows)
        od = d.step_dense(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows, map_len)
        if int(h.CNT[:, oracle.LOST_COLLISION].sum() + h.CNT[:, oracle.LOST_EXHAUSTED].sum()):
            break
        assert np.array_equal(oh.slot_table, od.slot_table)
        assert np.array_equal(oh.hit_mask, od.hit_mask)
        assert np.array_equal(oh.n_miss, od.n_miss)
        assert np.array_equal(h.C, d.C) and np.array_equal(h.F, d.F)
        for k in (oracle.HITS, oracle.LOOKUPS, oracle.MISSES, oracle.LIVE_EVICTIONS,
                  oracle.ERRORS):
            assert np.array_equal(h.CNT[:, k], d.CNT[:, k])


@pytest.mark.parametrize("seed", range(30))
def test_dense_map_points_only_at_slots_that_cache_its_id(seed):
    """Invariant of the map: an entry x -> v is only ever kept while slot v
    caches x, and every cached id of a step without repeated ids is mapped
    (so hits are exactly the selected ids resident before the step)."""
    w = gen_fuzz(seed)
    o = Oracle.for_workload(w)
    map_len = int(w.host_rows.max())
    for t in range(w.steps):
        resident = [set(o.C[b][o.C[b] >= 0].tolist()) for b in range(w.B)]
        out = o.step_dense(w.topk[t], w.ctx_len[t], w.row_base, w.host_rows, map_len)
        for b in range(w.B):
            xs = np.flatnonzero(o.map[b] >= 0)
            assert (o.C[b][o.map[b][xs]] == xs).all()
            if not (o.CNT[b, oracle.ERRORS] & 2):
                cached = set(o.C[b][o.C[b] >= 0].tolist())
                assert cached == set(xs.tolist())
                if w.Nq == 1:
                    ids = w.topk[t, b, 0]
                    for i, x in enumerate(ids.tolist()):
                        if out.hit_mask[b, 0, i] >= 0:
                            assert bool(out.hit_mask[b, 0, i]) == (x in resident[b])


def test_dense_map_rejects_ids_past_its_length():
    """An id outside the map is reported like an out-of-range id: slot -1,
    flag -1 and error bit 1, and nothing is installed for it."""
    o = _oracle(K=4, S=8)
    out = o.step_dense(np.array([[[0, 5, 7, -1]]], np.int32), np.array([100], np.int32),
                       np.zeros(1, np.int64), np.array([100], np.int32), 6)
    assert out.slot_table[0, 0].tolist() == [0, 1, -1, -1]
    assert out.hit_mask[0, 0].tolist() == [0, 0, -1, -1]
    assert o.CNT[0, oracle.ERRORS] == 1 and out.n_miss[0, 0] == 2
    assert o.map[0].tolist() == [0, -1, -1, -1, -1, 1]
