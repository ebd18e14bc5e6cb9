"""Two independent pure-Python references used to pin the CPU oracle.

Both are written from the AVSG page ("AVSG: Accelerated Vectorized Sparse
Gather for Efficient KV Cache Offload in Sparse-Attention LLM Serving"),
structured differently from the oracle on purpose, and only fit tiny inputs.

``brute_step`` transcribes the method literally, without shortcuts:
  * the Probe primitive examines *every* one of the R+1 buckets (section 3.3)
    and the smallest matching round is taken afterwards;
  * the hash is evaluated in exact integer arithmetic, ``(a1*x) % S``;
  * the extra decay of section 3.3, which continues until enough records have
    died, is run as repeated unit decays rather than a computed amount;
  * every reusable round of the link probe is listed, then the first taken;
    contested buckets are resolved by grouping claims per bucket (App. B,
    "Collision and probe-budget semantics").

``DictSim`` is a sequential LRU-with-aging simulator with *no hash table at
all*: an exact id -> slot dictionary plus the per-slot lifetimes of section
3.5.  Whenever the oracle has lost no bucket mapping, the two must agree on
everything the dictionary can see; this pins the hash layer as an exact
dictionary and the aging rule independently.
"""
from __future__ import annotations

import numpy as np

EMPTY = -1


class BruteState:
    def __init__(self, B, S):
        self.Q = [[EMPTY] * S for _ in range(B)]
        self.C = [[-1] * S for _ in range(B)]
        self.F = [[-1] * S for _ in range(B)]
        self.CNT = [[0] * 8 for _ in range(B)]


def _fp(x, afp):
    return ((x * afp) % (1 << 32)) // (1 << 17)


def _word(x, slot, afp):
    return _fp(x, afp) * 65536 + slot


def _buckets(x, S, R, a1, a2):
    h = (a1 * x) % S
    d = ((a2 * x) % S) | 1
    return [(h + t * d) % S for t in range(R + 1)]


def brute_step(st, p, topk, ctx_len, row_base, host_rows, host_rows_total):
    """One step on BruteState ``st``; returns (O, HIT, n, pairs) as lists."""
    B, Nq, K, S, L, R = p["B"], p["Nq"], p["K"], p["S"], p["L"], p["R"]
    a1, a2, afp = p["a1"], p["a2"], p["afp"]
    O = [[[-1] * K for _ in range(Nq)] for _ in range(B)]
    HIT = [[[-1] * K for _ in range(Nq)] for _ in range(B)]
    n = [[0] * Nq for _ in range(B)]
    pairs = [[[] for _ in range(Nq)] for _ in range(B)]
    for b in range(B):
        Q, C, F, cnt = st.Q[b], st.C[b], st.F[b], st.CNT[b]
        ok_row = (row_base[b] >= 0 and host_rows[b] >= 0
                  and row_base[b] + host_rows[b] <= host_rows_total)
        F[:] = [max(f - 1, -1) for f in F]
        for g in range(Nq):
            X = [int(v) for v in topk[b][g]]
            valid = []
            for i, x in enumerate(X):
                if x == -1:
                    continue
                if not ok_row or x < 0 or x >= host_rows[b]:
                    cnt[6] |= 1
                    continue
                valid.append(i)
            hit_slot = {}
            for i in valid:
                x = X[i]
                rounds = [t for t, q in enumerate(_buckets(x, S, R, a1, a2))
                          if Q[q] != EMPTY and C[Q[q] % 65536] == x]
                if rounds:
                    t = min(rounds)
                    hit_slot[i] = Q[_buckets(x, S, R, a1, a2)[t]] % 65536
                    cnt[7] += t + 1
                else:
                    cnt[7] += R + 1
            for i, s in hit_slot.items():
                F[s] = L
                O[b][g][i] = s
                HIT[b][g][i] = 1
            miss = sorted((X[i], i) for i in valid if i not in hit_slot)
            for r in range(1, len(miss)):
                if miss[r][0] == miss[r - 1][0]:
                    cnt[6] |= 2
            ng = len(miss)
            n[b][g] = ng
            if ng:
                while sum(1 for f in F if f == -1) < ng:
                    F[:] = [max(f - 1, -1) for f in F]
                victims = sorted(j for j in range(S) if F[j] == -1)[:ng]
                for r, ((x, i), v) in enumerate(zip(miss, victims)):
                    if C[v] >= 0:
                        cnt[5] += 1
                    C[v] = x
                    F[v] = L
                    O[b][g][i] = v
                    HIT[b][g][i] = 0
                    pairs[b][g].append((x, v))
                claims = {}
                for r, ((x, i), v) in enumerate(zip(miss, victims)):
                    reusable = []
                    for q in _buckets(x, S, R, a1, a2):
                        w = Q[q]
                        if w == EMPTY or C[w % 65536] == -1 or _fp(C[w % 65536], afp) != w // 65536:
                            reusable.append(q)
                    if not reusable:
                        cnt[4] += 1
                        continue
                    claims.setdefault(reusable[0], []).append((r, _word(x, v, afp)))
                for q, cl in claims.items():
                    cl.sort()
                    Q[q] = cl[-1][1]
                    cnt[3] += len(cl) - 1
            cnt[0] += len(hit_slot)
            cnt[1] += len(valid)
            cnt[2] += ng
        for j in range(S):
            if C[j] >= ctx_len[b]:
                C[j] = -1
    return O, HIT, n, pairs


class DictSim:
    """Exact-dictionary recall cache with per-slot aging (no hashing)."""

    def __init__(self, S, L):
        self.S, self.L = S, L
        self.slot_of = {}
        self.C = [-1] * S
        self.F = [-1] * S
        self.live_evictions = 0

    def step(self, tokens, ctx_len):
        """tokens: list of id lists (valid ids only).  Returns per token a
        dict id -> (slot, hit)."""
        S, L = self.S, self.L
        self.F = [max(f - 1, -1) for f in self.F]
        res = []
        for ids in tokens:
            out = {}
            for x in ids:
                if x in self.slot_of:
                    s = self.slot_of[x]
                    self.F[s] = L
                    out[x] = (s, 1)
            missing = sorted(x for x in ids if x not in out)
            while missing and self.F.count(-1) < len(missing):
                self.F = [max(f - 1, -1) for f in self.F]
            free = [j for j in range(S) if self.F[j] == -1]
            for x, v in zip(missing, free):
                old = self.C[v]
                if old >= 0:
                    self.live_evictions += 1
                    if self.slot_of.get(old) == v:
                        del self.slot_of[old]
                self.C[v] = x
                self.F[v] = L
                self.slot_of[x] = v
                out[x] = (v, 0)
            res.append(out)
        for j in range(S):
            if self.C[j] >= ctx_len:
                old = self.C[j]
                if self.slot_of.get(old) == j:
                    del self.slot_of[old]
                self.C[j] = -1
        return res


def as_np_state(st):
    return (np.array(st.Q, np.int32), np.array(st.C, np.int32),
            np.array(st.F, np.int32), np.array(st.CNT, np.int64))
