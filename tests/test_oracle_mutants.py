"""Mutation check of the oracle's pins (CPU only).

Each case plants one plausible mistake in a scratch copy of the oracle's C
source: a dropped term, a flipped comparison, a wrong order or index.  It
builds the copy with gcc into a temporary directory and runs the pins
(tests/test_oracle_pins.py) against that library.  The pins must fail for
every mutant.  A clean copy built the same way must pass, which shows that
the library swap itself works.  Nothing here touches the committed oracle
or the GPU library.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "avsg_oracle.c")
PINS = os.path.join(HERE, "test_oracle_pins.py")

# (name, text to replace, replacement, which occurrence: 0 = first, -1 = last).
# The main matcher comes first in the file, then the dense map, the
# no-reuse mode, the sort-merge matcher and the prefetch.
MUTANTS = [
    ("pre-decay dropped",
     "for (int32_t j = 0; j < S; ++j) F[j] = max32(F[j] - 1, -1);", "(void)0;", 0),
    ("highest-index victims",
     "for (int32_t j = 0; j < S && nv < n_g; ++j)",
     "for (int32_t j = S - 1; j >= 0 && nv < n_g; --j)", 0),
    ("F <= k instead of F < k in the extra decay",
     "below += (F[j] < kstar);", "below += (F[j] <= kstar);", 0),
    ("smallest rank keeps a contested bucket",
     "for (int32_t r = 0; r < n_g; ++r)\n                    if (target[r] >= 0)\n"
     "                        Q[target[r]] = pack_word",
     "for (int32_t r = n_g - 1; r >= 0; --r)\n                    if (target[r] >= 0)\n"
     "                        Q[target[r]] = pack_word", 0),
    ("> instead of >= in the invalidation",
     "if (C[j] >= ctx_len[b]) C[j] = -1;", "if (C[j] > ctx_len[b]) C[j] = -1;", 0),
    ("no refresh of hits", "F[found[i]] = L;", "(void)0;", 0),
    ("even probe stride", "% (uint32_t)c->S) | 1u;", "% (uint32_t)c->S) & ~1u;", 0),
    ("bucket of an empty slot not reusable",
     "if (cached == -1) return 1;", "if (cached == -1) return 0;", 0),
    ("stale fingerprint not reusable",
     "return fingerprint(c, cached) != word_fp(w);",
     "return fingerprint(c, cached) != word_fp(w) && 0;", 0),
    ("R rounds instead of R + 1", "for (int32_t t = 0; t <= c->R; ++t) {",
     "for (int32_t t = 0; t < c->R; ++t) {", 0),
    ("misses in descending id", "return p->id < q->id ? -1 : 1;",
     "return p->id < q->id ? 1 : -1;", 0),
    ("16-bit fingerprint shift", ">> 17);", ">> 16);", 0),
    ("live eviction of slot 0's id not counted",
     "if (C[v] >= 0) ++live_ev;", "if (C[v] > 0) ++live_ev;", 0),
    ("exhausted links not counted", "if (target[r] < 0) ++lost_exh;", "(void)0;", 0),
    ("dense: invalidation keeps the map entry",
     "if (C[j] >= 0 && C[j] < map_len && map[C[j]] == j) map[C[j]] = -1;", "(void)0;", 0),
    ("dense: install does not map the new id", "map[x] = v;", "(void)0;", 0),
    ("dense: pre-decay dropped",
     "for (int32_t j = 0; j < S; ++j) F[j] = max32(F[j] - 1, -1);", "(void)0;", -1),
    ("no-reuse: slot ignores the token", "O[i] = g * K + i;", "O[i] = i;", 0),
    ("sort-merge: referenced rows reset for each token",
     "memset(referenced, 0, (size_t)S);\n        for (int32_t g = 0; g < Nq; ++g) {",
     "for (int32_t g = 0; g < Nq; ++g) {\n        memset(referenced, 0, (size_t)S);", 0),
    ("sort-merge: an id cached twice hits the higher row",
     "for (int32_t j = 0; j < S; ++j)\n                    if (C[j] == x) { row = j; break; }",
     "for (int32_t j = S - 1; j >= 0; --j)\n                    if (C[j] == x) { row = j; break; }",
     0),
    ("sort-merge: a token's hits free for its own misses",
     "if (H[i] == 1) referenced[O[i]] = 1;", "(void)0;", 0),
    ("sort-merge: > instead of >= in the invalidation",
     "if (C[j] >= ctx_len[b]) C[j] = -1;", "if (C[j] > ctx_len[b]) C[j] = -1;", -1),
    ("prefetch: >= theta", "> theta[b]) out[m++]", ">= theta[b]) out[m++]", 0),
    ("threshold: weights swapped", "(1.0f - alpha) * theta[b]", "alpha * theta[b]", 0),
]


def _mutate(text: str, old: str, new: str, which: int) -> str:
    n = text.count(old)
    assert n >= 1, f"mutation target not found: {old!r}"
    idx = -1
    for _ in range(n if which == -1 else which + 1):
        idx = text.index(old, idx + 1)
    return text[:idx] + new + text[idx + len(old):]


def _run_pins(lib: str) -> subprocess.CompletedProcess:
    env = dict(os.environ, AVSG_ORACLE_LIB=lib)
    return subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q",
                           "-p", "no:cacheprovider", "-p", "no:randomly"],
                          cwd=os.path.dirname(HERE), env=env, capture_output=True,
                          text=True, timeout=600)


def _build(tmp, name: str, text: str) -> str:
    src = os.path.join(tmp, name + ".c")
    with open(src, "w") as f:
        f.write(text)
    return oracle.build(src=src, out=os.path.join(tmp, name + ".so"))


def test_every_planted_mistake_fails_a_pin(tmp_path):
    with open(SRC) as f:
        text = f.read()
    tmp = str(tmp_path)
    clean = _run_pins(_build(tmp, "clean", text))
    assert clean.returncode == 0, clean.stdout[-3000:]
    libs = [_build(tmp, f"m{i}", _mutate(text, old, new, which))
            for i, (_, old, new, which) in enumerate(MUTANTS)]
    with ThreadPoolExecutor(max_workers=4) as ex:
        runs = list(ex.map(_run_pins, libs))
    survivors = [name for (name, *_), r in zip(MUTANTS, runs)
                 if r.returncode in (0, 2, 3, 4, 5)]
    assert not survivors, f"mutants no pin caught: {survivors}"


@pytest.mark.parametrize("which", [0, -1])
def test_mutation_helper_replaces_the_chosen_occurrence(which):
    out = _mutate("a x b x c", "x", "Y", which)
    assert out == ("a Y b x c" if which == 0 else "a x b Y c")
