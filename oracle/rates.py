"""Rate definitions used to report the recall path's behaviour.

TEST INFRASTRUCTURE ONLY (imported by tests and the benchmark's reporting).

Each definition restates one the AVSG page uses:
  - hit rate: hits over valid lookups (section 4.4, buffer hit rates);
  - adjacent-step reuse: the fraction of the current selection that the
    preceding step also selected (section 4.4);
  - reuse rate: one minus the copies made over the lookups made, the form in
    which section 4.4 turns 61.87 % MTP-3 reuse into 8192*(1-61.87 %) copies;
  - gain: the 8K-buffer hit rate minus adjacent-step reuse, in percentage
    points (section 4.4, Table 1 caption).
"""
from __future__ import annotations

import numpy as np


def hit_rate(hits: int, lookups: int) -> float:
    return hits / lookups if lookups else 0.0


def reuse_rate(copies: int, lookups: int) -> float:
    return 1.0 - copies / lookups if lookups else 0.0


def copies_at_reuse(lookups: int, reuse: float) -> float:
    return lookups * (1.0 - reuse)


def gain_pp(hit_rate_pct: float, adjacent_reuse_pct: float) -> float:
    return hit_rate_pct - adjacent_reuse_pct


def adjacent_reuse(prev_ids, cur_ids) -> float:
    prev = {int(x) for x in np.asarray(prev_ids).ravel() if x >= 0}
    cur = [int(x) for x in np.asarray(cur_ids).ravel() if x >= 0]
    return sum(1 for x in cur if x in prev) / len(cur) if cur else 0.0


def latency_reduction(before: float, after: float) -> float:
    return 1.0 - after / before
