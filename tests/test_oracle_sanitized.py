"""The oracle's pins under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only).

The oracle is built with ``-fsanitize=address,undefined`` into a temporary
directory, and the pin suite runs against it in a child process that has
the gcc sanitizer runtimes preloaded.  Any out-of-bounds access, use of
freed memory, signed overflow or shift out of range aborts that process.
A second child runs a copy with a planted out-of-bounds read (the dense
map's invalidation without its id >= 0 check) on an input that reaches it.
That read must be reported, which shows the sanitizers are live.
"""
from __future__ import annotations

import os
import subprocess
import sys

import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(ROOT, "oracle", "avsg_oracle.c")


def _runtime(name):
    try:
        path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                              text=True, check=True).stdout.strip()
    except (OSError, subprocess.CalledProcessError):
        return None
    return path if os.path.isabs(path) and os.path.exists(path) else None


ASAN, UBSAN = _runtime("libasan.so"), _runtime("libubsan.so")
pytestmark = pytest.mark.skipif(not (ASAN and UBSAN),
                                reason="gcc's sanitizer runtimes are not installed")


def _env(lib):
    return dict(os.environ, AVSG_ORACLE_LIB=lib, LD_PRELOAD=f"{ASAN}:{UBSAN}",
                ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
                UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def test_pins_pass_under_sanitizers(tmp_path):
    lib = oracle.build(out=str(tmp_path / "liboracle_san.so"), sanitize=True)
    r = subprocess.run([sys.executable, "-m", "pytest",
                        os.path.join(HERE, "test_oracle_pins.py"),
                        os.path.join(HERE, "test_workloads.py"),
                        "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=_env(lib), capture_output=True, text=True, timeout=900)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "Sanitizer" not in out and "runtime error" not in out, out[-4000:]


PLANTED = """
import numpy as np
from oracle import Oracle
o = Oracle(1, 1, 4, 16, 3, 7, 1, 3, 5, 16, 100)
o.step_dense(np.array([[[1, 2, 3, 4]]], np.int32), np.array([-1], np.int32),
             np.zeros(1, np.int64), np.array([100], np.int32), 100)
print("finished")
"""


def test_a_planted_out_of_bounds_read_is_reported(tmp_path):
    with open(SRC) as f:
        text = f.read()
    good = "if (C[j] >= 0 && C[j] < map_len && map[C[j]] == j) map[C[j]] = -1;"
    assert text.count(good) == 1
    src = tmp_path / "planted.c"
    src.write_text(text.replace(good, "if (C[j] < map_len && map[C[j]] == j) map[C[j]] = -1;"))
    lib = oracle.build(src=str(src), out=str(tmp_path / "libplanted.so"), sanitize=True)
    env = _env(lib)
    env["PYTHONPATH"] = ROOT
    r = subprocess.run([sys.executable, "-c", PLANTED], cwd=ROOT, env=env,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 and "heap-buffer-overflow" in r.stderr, r.stderr[-3000:]
    assert "finished" not in r.stdout
