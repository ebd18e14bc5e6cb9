"""Seeded synthetic inputs for the per-decode-step KV recall path.

This module only *draws inputs*: the top-K token indices each query token
selects, the verified context length of each request, where each request's
rows sit in the host KV pool, and the bytes of that pool.  It holds none of
the recall method's arithmetic (no hashing, probing, aging or slot choice),
which is why both the CPU oracle and the GPU path may read from it.

The pages measure on production agent requests, the ServeGen / Mooncake
traces and real model weights, none of which are available here.  These
generators stand in for them with the shapes the pages describe: a sparse
indexer picks K = 2048 earlier tokens per query token (AVSG page, section 1
and section 2 on DSA), selections drift between adjacent decode steps
(AVSG page, section 4.4), MTP iterations carry one initial and several
speculative tokens (AVSG page, section 3.6), and request lengths are
long-tailed (PulseInfer page, section 3.3 on request-length CDFs).

Every generator is a pure function of its seed: ``numpy.random.default_rng``
seeded with ``[config_seed, request]`` per request, so requests can be drawn
independently and in any order.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

# Hash constants handed to both sides as plain configuration values.  The
# pages do not print them (AVSG page, section 3.3, "Probe primitive"); any odd
# 32-bit values are admissible.
DEFAULT_A1 = 0x9E3779B1
DEFAULT_A2 = 0x85EBCA77
DEFAULT_AFP = 0xC2B2AE3D
DEFAULT_L = 15
DEFAULT_R = 7

CONFIG_NAMES = ("tiny", "matching", "residency", "mtp3", "imbalanced")
CONFIG_SEEDS = {"tiny": 101, "matching": 202, "residency": 303, "mtp3": 404,
                "imbalanced": 505}

_KV_CHUNK = 64 << 20  # host KV bytes are drawn in independent 64 MiB chunks


@dataclass
class Workload:
    """One synthetic recall workload: shapes plus every step's inputs.

    topk      int32 [steps][B][Nq][K]   selected token ids, -1 = padding
    ctx_len   int32 [steps][B]          verified context length N per request
    host_rows int32 [B]                 valid host rows of each request
    row_base  int64 [B]                 first host row of each request
    """
    name: str
    B: int
    Nq: int
    K: int
    S: int
    row_bytes: int
    steps: int
    seed: int
    topk: np.ndarray
    ctx_len: np.ndarray
    host_rows: np.ndarray
    row_base: np.ndarray
    L: int = DEFAULT_L
    R: int = DEFAULT_R
    a1: int = DEFAULT_A1
    a2: int = DEFAULT_A2
    afp: int = DEFAULT_AFP
    extra: dict = field(default_factory=dict)

    @property
    def host_rows_total(self) -> int:
        return int(self.row_base[-1] + self.host_rows[-1]) if self.B else 0

    @property
    def host_bytes(self) -> int:
        return self.host_rows_total * self.row_bytes

    @property
    def lookups_per_step(self) -> int:
        return self.B * self.Nq * self.K

    def params(self) -> dict:
        return dict(B=self.B, Nq=self.Nq, K=self.K, S=self.S, L=self.L,
                    R=self.R, a1=self.a1, a2=self.a2, afp=self.afp,
                    row_bytes=self.row_bytes)

    def fill_host_kv(self, out: np.ndarray) -> None:
        """Fill ``out`` (uint8, host_bytes long) with the pool's bytes."""
        fill_random_bytes(out, self.seed)


def fill_random_bytes(out: np.ndarray, seed: int) -> None:
    """Uniform random bytes, drawn chunk by chunk from ``[seed, 9999, chunk]``."""
    flat = out.reshape(-1)
    assert flat.dtype == np.uint8
    n = flat.size
    for c, lo in enumerate(range(0, n, _KV_CHUNK)):
        hi = min(n, lo + _KV_CHUNK)
        rng = np.random.default_rng([seed, 9999, c])
        flat[lo:hi] = np.frombuffer(rng.bytes(hi - lo), dtype=np.uint8)


# ---------------------------------------------------------------- helpers --

def _take_distinct(rng, need, draw, taken):
    """Collect ``need`` distinct ids from ``draw(size)``, skipping ``taken``.

    ``taken`` is a boolean mask over the id domain; accepted ids are marked in
    it.  Ids are accepted in the order they are drawn.
    """
    got = []
    have = 0
    while have < need:
        cand = draw(max(2 * (need - have), 256))
        cand = cand[~taken[cand]]
        if cand.size == 0:
            continue
        _, first = np.unique(cand, return_index=True)
        cand = cand[np.sort(first)][: need - have]
        taken[cand] = True
        got.append(cand)
        have += cand.size
    return np.concatenate(got).astype(np.int64) if got else np.zeros(0, np.int64)


def _zipf_sampler(rng, perm, s=1.1):
    """Ids = perm[rank-1] with rank ~ Zipf(s), ranks beyond len(perm) rejected."""
    limit = perm.size

    def draw(size):
        r = rng.zipf(s, size=size)
        r = r[r <= limit]
        return perm[r - 1]
    return draw


def _uniform_sampler(rng, hi):
    def draw(size):
        return rng.integers(0, hi, size=size)
    return draw


def _as_row(ids, K):
    out = np.full(K, -1, np.int32)
    out[: ids.size] = ids
    return out


# ------------------------------------------------------------ the configs --

def gen_tiny(steps=16):
    """1 request, context 4096, K=256, S=512, 1152-B rows (576 bf16).

    Step 0 draws 256 distinct ids uniformly from [0, 4096).  Each later step
    keeps round(0.7*256) = 179 of the previous ids, chosen uniformly, and adds
    77 new distinct ids drawn uniformly from [0, 4096) minus the kept ones.
    Ids are emitted sorted ascending.
    """
    seed, ctx, K = CONFIG_SEEDS["tiny"], 4096, 256
    B, Nq = 1, 1
    keep = int(round(0.7 * K))
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    for b in range(B):
        rng = np.random.default_rng([seed, b])
        prev = None
        for t in range(steps):
            if prev is None:
                ids = rng.choice(ctx, K, replace=False)
            else:
                kept = rng.choice(prev, keep, replace=False)
                taken = np.zeros(ctx, bool)
                taken[kept] = True
                new = _take_distinct(rng, K - keep, _uniform_sampler(rng, ctx), taken)
                ids = np.concatenate([kept, new])
            ids = np.sort(ids)
            topk[t, b, 0] = ids
            prev = ids
    return Workload("tiny", B, Nq, K, 512, 1152, steps, seed, topk,
                    np.full((steps, B), ctx, np.int32), np.full(B, ctx, np.int32),
                    np.arange(B, dtype=np.int64) * ctx)


def _window_plus_zipf(rng, perm, ctx, K, win):
    window = np.arange(ctx - win, ctx)
    taken = np.zeros(ctx, bool)
    taken[window] = True
    z = _take_distinct(rng, K - win, _zipf_sampler(rng, perm), taken)
    return window, z


def gen_matching(steps=64, layer=0):
    """Batch 8, context 65536, K=2048, S=2048, 1280-B rows (576 bf16 + 128 fp8).

    Every step selects the 256-token recency window [ctx-256, ctx) plus 1792
    distinct ids whose Zipf(s=1.1) ranks are mapped through a per-request
    random permutation of [0, ctx-256) (fixed per request, so low ranks form
    a hot set); the Zipf draws are redrawn every step.  Ids are emitted in
    random order.  ``layer`` > 0 draws another layer's selections for the
    same requests (independent streams; layer 0 is the matching workload).
    """
    seed, ctx, K, win = CONFIG_SEEDS["matching"], 65536, 2048, 256
    B, Nq = 8, 1
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    for b in range(B):
        rng = np.random.default_rng([seed, b] if layer == 0 else [seed, b, layer])
        perm = rng.permutation(ctx - win)
        for t in range(steps):
            window, z = _window_plus_zipf(rng, perm, ctx, K, win)
            topk[t, b, 0] = rng.permutation(np.concatenate([window, z]))
    return Workload("matching", B, Nq, K, 2048, 1280, steps, seed, topk,
                    np.full((steps, B), ctx, np.int32), np.full(B, ctx, np.int32),
                    np.arange(B, dtype=np.int64) * ctx)


def gen_residency(steps=128, B=32):
    """Batch 32, context 131072, K=2048, S=8192, 1280-B rows, 15 % drift.

    Step 0 is drawn as in the matching workload.  Each later step keeps the
    recency window, keeps 1792-307 = 1485 of the previous step's non-window
    ids (uniformly chosen) and replaces round(0.15*2048) = 307 of them with
    fresh Zipf draws not already selected, so adjacent-step reuse is about
    85 % by construction.  Ids are emitted in random order.
    """
    seed, ctx, K, win = CONFIG_SEEDS["residency"], 131072, 2048, 256
    Nq = 1
    repl = int(round(0.15 * K))
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    for b in range(B):
        rng = np.random.default_rng([seed, b])
        perm = rng.permutation(ctx - win)
        window, z = _window_plus_zipf(rng, perm, ctx, K, win)
        for t in range(steps):
            if t > 0:
                kept = rng.choice(z, z.size - repl, replace=False)
                taken = np.zeros(ctx, bool)
                taken[window] = True
                taken[kept] = True
                fresh = _take_distinct(rng, repl, _zipf_sampler(rng, perm), taken)
                z = np.concatenate([kept, fresh])
            topk[t, b, 0] = rng.permutation(np.concatenate([window, z]))
    return Workload("residency", B, Nq, K, 8192, 1280, steps, seed, topk,
                    np.full((steps, B), ctx, np.int32), np.full(B, ctx, np.int32),
                    np.arange(B, dtype=np.int64) * ctx)


def gen_mtp3(steps=32, B=16):
    """Batch 16, 4 query tokens per iteration (1 initial + 3 speculative).

    Iteration t has verified length N_t = 100000 - 128 + 4t.  Token g selects
    the window [N_t+g-256, N_t+g) (so tokens g >= 1 also select the
    speculative positions [N_t, N_t+g)).  Token 0 adds 1792 distinct Zipf ids
    over a per-request permutation of [0, 99616); token g >= 1 keeps
    round(0.6*1792) = 1075 of them (uniformly chosen) and adds 717 fresh Zipf
    ids not among token 0's.  Host rows exist for all positions < 100000.
    The buffer starts empty.
    """
    seed, ctx, K, win, Nq = CONFIG_SEEDS["mtp3"], 100000, 2048, 256, 4
    base = ctx - 128
    dom = base - win
    n_z = K - win
    keep = int(round(0.6 * n_z))
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    ctx_len = np.zeros((steps, B), np.int32)
    for b in range(B):
        rng = np.random.default_rng([seed, b])
        perm = rng.permutation(dom)
        for t in range(steps):
            N = base + 4 * t
            ctx_len[t, b] = N
            taken0 = np.zeros(dom, bool)
            z0 = _take_distinct(rng, n_z, _zipf_sampler(rng, perm), taken0)
            for g in range(Nq):
                window = np.arange(N + g - win, N + g)
                if g == 0:
                    z = z0
                else:
                    kept = rng.choice(z0, keep, replace=False)
                    taken = taken0.copy()
                    fresh = _take_distinct(rng, n_z - keep, _zipf_sampler(rng, perm), taken)
                    z = np.concatenate([kept, fresh])
                topk[t, b, g] = rng.permutation(np.concatenate([window, z]))
    return Workload("mtp3", B, Nq, K, 8192, 1280, steps, seed, topk, ctx_len,
                    np.full(B, ctx, np.int32), np.arange(B, dtype=np.int64) * ctx)


def gen_imbalanced(steps=64, B=64):
    """64 requests with lognormal lengths, S=4096, 1280-B rows.

    len_b = clip(round(16384 * exp(z_b)), 2048, 262144) with z_b ~ N(0, 1)
    (median 16K); per-request drift r_b ~ U(0, 0.6).  K_b = min(2048, len_b)
    = 2048.  Step 0 draws K distinct ids uniformly from [0, len_b); each later
    step keeps round((1-r_b)*K) of the previous ids and draws the rest
    uniformly from [0, len_b) minus the kept ones.  Host rows are packed:
    row_base[b] = sum of earlier lengths.  Ids are emitted in random order.
    """
    seed, K = CONFIG_SEEDS["imbalanced"], 2048
    Nq = 1
    rl = np.random.default_rng([seed, 7777])
    z = rl.standard_normal(B)
    lens = np.clip(np.round(16384 * np.exp(z)), 2048, 262144).astype(np.int64)
    drift = rl.uniform(0.0, 0.6, B)
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    for b in range(B):
        rng = np.random.default_rng([seed, b])
        n = int(lens[b])
        kb = min(K, n)
        keep = int(round((1.0 - drift[b]) * kb))
        prev = None
        for t in range(steps):
            if prev is None:
                ids = rng.choice(n, kb, replace=False)
            else:
                kept = rng.choice(prev, keep, replace=False)
                taken = np.zeros(n, bool)
                taken[kept] = True
                new = _take_distinct(rng, kb - keep, _uniform_sampler(rng, n), taken)
                ids = np.concatenate([kept, new])
            ids = rng.permutation(ids)
            topk[t, b, 0] = _as_row(ids, K)
            prev = ids
    row_base = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    ctx = np.broadcast_to(lens.astype(np.int32), (steps, B)).copy()
    w = Workload("imbalanced", B, Nq, K, 4096, 1280, steps, seed, topk, ctx,
                 lens.astype(np.int32), row_base)
    w.extra["drift"] = drift
    return w


def gen_reuse(B, reuse, steps=16, name=None, seed=606, K=2048, S=4096):
    """Fixed adjacent-step reuse, for the transfer-partition comparison the
    AVSG page makes at B = 1 with 25 % reuse and at B = 8 with 75 % reuse
    (section 4.3), and for matching latency against K and S (section 4.2):
    context 65536, K = 2048 and S = 4096 unless given, 1280-B rows.

    Step 0 draws K distinct ids uniformly; each later step keeps
    round(reuse * K) of the previous ids (chosen uniformly) and adds fresh
    distinct ids drawn uniformly from the rest of the context.  Ids are
    emitted in random order.
    """
    ctx = 65536
    Nq = 1
    keep = int(round(reuse * K))
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    for b in range(B):
        rng = np.random.default_rng([seed, int(round(reuse * 100)), b])
        prev = None
        for t in range(steps):
            if prev is None:
                ids = rng.choice(ctx, K, replace=False)
            else:
                kept = rng.choice(prev, keep, replace=False)
                taken = np.zeros(ctx, bool)
                taken[prev] = True
                new = _take_distinct(rng, K - keep, _uniform_sampler(rng, ctx), taken)
                ids = np.concatenate([kept, new])
            ids = rng.permutation(ids)
            topk[t, b, 0] = ids
            prev = ids
    name = name or f"reuse{int(round(reuse * 100))}_b{B}"
    return Workload(name, B, Nq, K, S, 1280, steps, seed, topk,
                    np.full((steps, B), ctx, np.int32), np.full(B, ctx, np.int32),
                    np.arange(B, dtype=np.int64) * ctx)


def gen_skewed_reuse(B=8, lo=0.4, hi=1.0, steps=16, seed=808, K=2048, S=4096):
    """Per-request adjacent-step reuse spread over [lo, hi], so per-request
    miss rates spread over 0-60 % as in the imbalanced workload, at the
    matching batch of 8 (the transfer-partition comparison of the AVSG page,
    section 4.3, where uneven misses are what a per-row split balances):
    context 65536, K = 2048, S = 4096, 1280-B rows.

    Request b keeps round(r_b * K) of its previous ids each step.  The r_b
    are B evenly spaced values from lo to hi, in an order shuffled by
    ``default_rng([seed, 7777])``, so a small batch spans the whole range.
    Otherwise as ``gen_reuse``.
    """
    ctx = 65536
    Nq = 1
    reuse = np.random.default_rng([seed, 7777]).permutation(np.linspace(lo, hi, B))
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    for b in range(B):
        rng = np.random.default_rng([seed, b])
        keep = int(round(reuse[b] * K))
        prev = None
        for t in range(steps):
            if prev is None:
                ids = rng.choice(ctx, K, replace=False)
            else:
                kept = rng.choice(prev, keep, replace=False)
                taken = np.zeros(ctx, bool)
                taken[prev] = True
                new = _take_distinct(rng, K - keep, _uniform_sampler(rng, ctx), taken)
                ids = np.concatenate([kept, new])
            ids = rng.permutation(ids)
            topk[t, b, 0] = ids
            prev = ids
    w = Workload(f"skew{int(round(lo * 100))}to{int(round(hi * 100))}_b{B}", B, Nq, K, S,
                 1280, steps, seed, topk, np.full((steps, B), ctx, np.int32),
                 np.full(B, ctx, np.int32), np.arange(B, dtype=np.int64) * ctx)
    w.extra["reuse"] = reuse
    return w


def stack_layers(ws, name=None):
    """One workload whose requests are the (layer, request) pairs of the
    per-layer workloads ``ws`` (same shapes): each layer keeps its own cache
    and its own host rows, so the stacked batch is layer-major, B' = L * B,
    and layer l's rows sit after those of layers < l in one host pool."""
    w0 = ws[0]
    L = len(ws)
    topk = np.concatenate([w.topk for w in ws], axis=1)
    ctx = np.concatenate([w.ctx_len for w in ws], axis=1)
    host_rows = np.concatenate([w.host_rows for w in ws])
    per_layer = w0.host_rows_total
    row_base = np.concatenate([w.row_base + l * per_layer for l, w in enumerate(ws)])
    return Workload(name or f"{w0.name}x{L}", w0.B * L, w0.Nq, w0.K, w0.S, w0.row_bytes,
                    w0.steps, w0.seed, topk, ctx, host_rows.astype(np.int32),
                    row_base.astype(np.int64), L=w0.L, R=w0.R, a1=w0.a1, a2=w0.a2,
                    afp=w0.afp)


def gen_scored(B=8, steps=32, noise=0.3, seed=707):
    """Indexer scores and their exact top-K, for threshold prefetch (ECHO
    page, decode prefetch): context 65536, K = 2048, S = 4096 (room for a
    prefetch token ahead of the exact one), 1280-B rows.

    Each request has a fixed relevance over a random permutation of the
    context, -0.8 * log(1 + rank / 8) (a hot head and a long tail), plus 10
    on the 256 most recent tokens.  Step t scores every token as relevance
    plus Gaussian noise (sd ``noise``, 0.3 giving about 82 % adjacent-step
    reuse of the top-K, near the 81.61 % the AVSG page reports), in float32.
    The selection is the exact top-K of the scores (random order), and the
    K-th highest score is kept for the threshold.
    """
    ctx, K, S = 65536, 2048, 4096
    Nq = 1
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    scores = np.empty((steps, B, ctx), np.float32)
    kth = np.empty((steps, B), np.float32)
    for b in range(B):
        rng = np.random.default_rng([seed, b])
        perm = rng.permutation(ctx)
        base = np.empty(ctx, np.float32)
        base[perm] = (-0.8 * np.log1p(np.arange(ctx) / 8.0)).astype(np.float32)
        base[ctx - 256:] += np.float32(10.0)
        for t in range(steps):
            sc = base + (noise * rng.standard_normal(ctx)).astype(np.float32)
            part = np.argpartition(-sc, K - 1)
            top = part[:K]
            scores[t, b] = sc
            kth[t, b] = sc[part[K - 1]]
            topk[t, b, 0] = rng.permutation(top)
    w = Workload("scored", B, Nq, K, S, 1280, steps, seed, topk,
                 np.full((steps, B), ctx, np.int32), np.full(B, ctx, np.int32),
                 np.arange(B, dtype=np.int64) * ctx)
    w.extra["scores"] = scores
    w.extra["kth"] = kth
    return w


def gen_reuse25_b1(steps=16):
    return gen_reuse(1, 0.25, steps)


def gen_reuse75_b8(steps=16):
    return gen_reuse(8, 0.75, steps)


GENERATORS = {"tiny": gen_tiny, "matching": gen_matching,
              "residency": gen_residency, "mtp3": gen_mtp3,
              "imbalanced": gen_imbalanced, "reuse25_b1": gen_reuse25_b1,
              "reuse75_b8": gen_reuse75_b8, "scored": gen_scored,
              "skew40to100_b8": gen_skewed_reuse}


def make(name: str, **kw) -> Workload:
    return GENERATORS[name](**kw)


# ----------------------------------------------------------- fuzz corpus --

def gen_fuzz(seed: int, steps: int = 6) -> Workload:
    """A small random case: B<=3, Nq<=3, K<=16, S in {16, 32, 64}.

    Ids come from a small universe so hits, evictions, lost mappings and
    speculative ids all occur.  Padding (-1), out-of-range ids and ids beyond
    the verified length are mixed in.  The capacity bound Nq*K <= S holds.
    """
    rng = np.random.default_rng([7, seed])
    S = int(rng.choice([16, 32, 64]))
    Nq = int(rng.integers(1, 4))
    K = int(rng.integers(1, min(16, S // Nq) + 1))
    B = int(rng.integers(1, 4))
    L = int(rng.choice([1, 2, 3, 5]))
    R = int(rng.choice([0, 1, 3, S - 1]))
    univ = int(rng.integers(K + 1, 6 * S))
    host_rows = rng.integers(max(1, univ // 2), univ + 1, size=B).astype(np.int32)
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    ctx = np.zeros((steps, B), np.int32)
    for t in range(steps):
        for b in range(B):
            hr = int(host_rows[b])
            ctx[t, b] = int(rng.integers(max(1, hr // 2), hr + 1))
            for g in range(Nq):
                n = int(rng.integers(0, min(K, hr) + 1))
                ids = rng.choice(hr, n, replace=False).astype(np.int32)
                row = np.full(K, -1, np.int32)
                pos = rng.permutation(K)[:n]
                row[pos] = ids
                # occasionally plant an out-of-range id in a padding position
                if n < K and rng.random() < 0.15:
                    free = np.setdiff1d(np.arange(K), pos)
                    row[free[0]] = int(rng.choice([-5, hr, hr + 3]))
                topk[t, b, g] = row
    row_base = np.concatenate([[0], np.cumsum(host_rows)[:-1]]).astype(np.int64)
    a1 = int(rng.integers(0, 2**31)) * 2 + 1
    a2 = int(rng.integers(0, 2**31)) * 2 + 1
    afp = int(rng.integers(0, 2**31)) * 2 + 1
    row_bytes = int(rng.choice([16, 32, 64]))
    return Workload(f"fuzz{seed}", B, Nq, K, S, row_bytes, steps, 1000 + seed,
                    topk, ctx, host_rows, row_base, L=L, R=R, a1=a1, a2=a2,
                    afp=afp)


def gen_medium(seed: int, steps: int = 3) -> Workload:
    """A random medium-sized case across the supported shapes.

    K in 1..4096 with N_q*K <= 8192, N_q in 1..4, S the smallest power of two
    >= N_q*K times 1, 2 or 4 (at most 16384), B up to 300 (more requests than CUs for small K),
    lookups per step kept under about 300k so the oracle stays fast.  Each
    token keeps about half of the request's previous selection and draws the
    rest fresh; padding, out-of-range ids and ids at or beyond the verified
    length are mixed in.  Rows are 16 to 64 bytes so the host pool stays small.
    """
    rng = np.random.default_rng([9, seed])
    Nq = int(rng.integers(1, 5))
    K = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(64, 1025)),
                        int(rng.integers(1024, 4097))]))
    K = max(1, min(K, 8192 // Nq))
    S = 16
    while S < Nq * K:
        S *= 2
    S = min(16384, S * int(rng.choice([1, 2, 4])))
    B = int(rng.integers(1, max(2, min(300, 300_000 // (Nq * K)) + 1)))
    L = int(rng.choice([1, 3, 15, 63]))
    R = int(rng.choice([0, 2, 7, min(15, S - 1)]))
    host_rows = rng.integers(max(K + 1, 2 * K), 8 * K + 64, size=B).astype(np.int32)
    topk = np.full((steps, B, Nq, K), -1, np.int32)
    ctx = np.zeros((steps, B), np.int32)
    prev = [None] * B
    for t in range(steps):
        for b in range(B):
            hr = int(host_rows[b])
            ctx[t, b] = int(rng.integers(max(1, (3 * hr) // 4), hr + 1))
            for g in range(Nq):
                n = K - int(rng.integers(0, max(1, K // 8) + 1))
                if prev[b] is not None and prev[b].size:
                    keep = rng.choice(prev[b], min(prev[b].size, n // 2), replace=False)
                else:
                    keep = np.empty(0, np.int64)
                fresh = np.setdiff1d(rng.choice(hr, min(hr, 2 * n), replace=False), keep)
                ids = np.concatenate([keep, fresh[: n - keep.size]]).astype(np.int32)
                prev[b] = ids
                row = np.full(K, -1, np.int32)
                row[rng.permutation(K)[: ids.size]] = rng.permutation(ids)
                if ids.size < K and rng.random() < 0.2:
                    free = np.flatnonzero(row == -1)
                    row[free[0]] = int(rng.choice([-7, hr, hr + 11]))
                topk[t, b, g] = row
    row_base = np.concatenate([[0], np.cumsum(host_rows)[:-1]]).astype(np.int64)
    a1 = int(rng.integers(0, 2**31)) * 2 + 1
    a2 = int(rng.integers(0, 2**31)) * 2 + 1
    afp = int(rng.integers(0, 2**31)) * 2 + 1
    row_bytes = int(rng.choice([16, 32, 64]))
    return Workload(f"medium{seed}", B, Nq, K, S, row_bytes, steps, 2000 + seed,
                    topk, ctx, host_rows, row_base, L=L, R=R, a1=a1, a2=a2, afp=afp)
