"""CPU oracle of the per-decode-step KV recall path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import this package.  The product
path (``recall_step_amd``) never imports it, and it never imports the
product: the two share nothing but the seeded input generators of
``workloads``.

The arithmetic lives in ``avsg_oracle.c`` (plain sequential C, compiled with
gcc); this module only marshals numpy arrays into it.  Pins for the oracle
(closed forms, a brute-force transcription, a dictionary simulator and the
pages' printed figures) are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "avsg_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

HITS, LOOKUPS, MISSES, LOST_COLLISION, LOST_EXHAUSTED, LIVE_EVICTIONS, \
    ERRORS, PROBE_VISITS = range(8)
ERR_OUT_OF_RANGE = 1
ERR_DUPLICATE = 2

RC_NAMES = {0: "ok", -1: "bad argument", -2: "slot referenced earlier in the "
            "step was evicted", -3: "lifetime out of range", -4: "out of memory"}


# Extra gcc flags of a sanitizer build (see build(sanitize=True)).
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build(src: str = _SRC, out: str = _LIB, sanitize: bool = False) -> str:
    """Compile the oracle source ``src`` with gcc into the shared library
    ``out`` (by default ``oracle/liboracle.so``).  ``sanitize`` builds it
    with AddressSanitizer and UndefinedBehaviorSanitizer; such a library is
    loaded by a process started with the sanitizer runtimes preloaded."""
    tmp = out + ".tmp"
    # -ffp-contract=off: float32 products and sums round one at a time.
    flags = ["-std=c11", "-Wall", "-Wextra", "-Werror", "-ffp-contract=off",
             "-shared", "-fPIC"]
    flags = (SANITIZE_FLAGS if sanitize else ["-O2"]) + flags
    subprocess.run(["gcc", *flags, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_lib = None


def library_path() -> str:
    """The library the wrapper loads: ``$AVSG_ORACLE_LIB`` when set (a
    sanitizer or test build made by build(); used as is, never rebuilt),
    else ``oracle/liboracle.so``, rebuilt when older than its source."""
    return os.environ.get("AVSG_ORACLE_LIB") or _LIB


def _load():
    global _lib
    if _lib is None:
        path = library_path()
        if path == _LIB and (not os.path.exists(_LIB) or
                             os.path.getmtime(_LIB) < os.path.getmtime(_SRC)):
            build()
        lib = ctypes.CDLL(path)
        p = ctypes.c_void_p
        lib.orc_step.argtypes = [p] * 15
        lib.orc_step.restype = ctypes.c_int
        lib.orc_step_no_reuse.argtypes = [p] * 11
        lib.orc_step_no_reuse.restype = ctypes.c_int
        lib.orc_step_dense.argtypes = [p, p, p, p, p, ctypes.c_int64] + [p] * 10
        lib.orc_step_dense.restype = ctypes.c_int
        lib.orc_step_sort_merge.argtypes = [p] * 13
        lib.orc_step_sort_merge.restype = ctypes.c_int
        lib.orc_prefetch_select.argtypes = [p, p, ctypes.c_int64, p, p, p, p]
        lib.orc_prefetch_select.restype = None
        lib.orc_ema_threshold.argtypes = [ctypes.c_int32, p, p, ctypes.c_float]
        lib.orc_ema_threshold.restype = None
        lib.orc_state_reset.argtypes = [p] * 5
        lib.orc_state_reset.restype = None
        lib.orc_version.restype = ctypes.c_int
        lib.orc_probe_buckets.argtypes = [p, ctypes.c_int32, p]
        lib.orc_probe_buckets.restype = None
        lib.orc_word.argtypes = [p, ctypes.c_int32, ctypes.c_int32]
        lib.orc_word.restype = ctypes.c_int32
        _lib = lib
    return _lib


class _Cfg(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("Nq", ctypes.c_int32),
                ("K", ctypes.c_int32), ("S", ctypes.c_int32),
                ("L", ctypes.c_int32), ("R", ctypes.c_int32),
                ("a1", ctypes.c_uint32), ("a2", ctypes.c_uint32),
                ("afp", ctypes.c_uint32), ("row_bytes", ctypes.c_int64),
                ("host_rows_total", ctypes.c_int64)]


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


@dataclass
class StepOut:
    slot_table: np.ndarray   # int32 [B][Nq][K]
    hit_mask: np.ndarray     # int8  [B][Nq][K]
    n_miss: np.ndarray       # int32 [B][Nq]
    miss_pairs: np.ndarray   # int32 [B][Nq][K][2]; rows >= n_miss are zero


class OracleError(RuntimeError):
    pass


class Oracle:
    """Stateful oracle: owns Q/C/F/CNT and the shadow device slot buffer."""

    def __init__(self, B, Nq, K, S, L, R, a1, a2, afp, row_bytes,
                 host_rows_total, host_kv=None, shadow=True):
        self.cfg = _Cfg(B, Nq, K, S, L, R, a1 & 0xFFFFFFFF, a2 & 0xFFFFFFFF,
                        afp & 0xFFFFFFFF, row_bytes, host_rows_total)
        self.B, self.Nq, self.K, self.S, self.L, self.R = B, Nq, K, S, L, R
        self.row_bytes = row_bytes
        self.Q = np.empty((B, S), np.int32)
        self.C = np.empty((B, S), np.int32)
        self.F = np.empty((B, S), np.int32)
        self.CNT = np.empty((B, 8), np.int32)
        self.host_kv = host_kv
        self.shadow = (np.zeros((B, S, row_bytes), np.uint8)
                       if (shadow and host_kv is not None) else None)
        self.reset()

    @classmethod
    def for_workload(cls, w, host_kv=None, shadow=True):
        return cls(w.B, w.Nq, w.K, w.S, w.L, w.R, w.a1, w.a2, w.afp,
                   w.row_bytes, w.host_rows_total, host_kv, shadow)

    def reset(self):
        self.map = None
        _load().orc_state_reset(ctypes.byref(self.cfg), _ptr(self.Q), _ptr(self.C),
                                _ptr(self.F), _ptr(self.CNT))

    def step(self, topk, ctx_len, row_base, host_rows) -> StepOut:
        B, Nq, K = self.B, self.Nq, self.K
        topk = np.ascontiguousarray(topk, np.int32).reshape(B, Nq, K)
        ctx_len = np.ascontiguousarray(ctx_len, np.int32).reshape(B)
        row_base = np.ascontiguousarray(row_base, np.int64).reshape(B)
        host_rows = np.ascontiguousarray(host_rows, np.int32).reshape(B)
        out = StepOut(np.empty((B, Nq, K), np.int32), np.empty((B, Nq, K), np.int8),
                      np.empty((B, Nq), np.int32), np.zeros((B, Nq, K, 2), np.int32))
        hk = self.host_kv
        if hk is not None:
            assert hk.dtype == np.uint8 and hk.flags.c_contiguous
        rc = _load().orc_step(ctypes.byref(self.cfg), _ptr(self.Q), _ptr(self.C),
                              _ptr(self.F), _ptr(self.CNT), _ptr(topk),
                              _ptr(ctx_len), _ptr(row_base), _ptr(host_rows),
                              _ptr(hk) if self.shadow is not None else None,
                              _ptr(self.shadow), _ptr(out.slot_table),
                              _ptr(out.hit_mask), _ptr(out.n_miss),
                              _ptr(out.miss_pairs))
        if rc != 0:
            raise OracleError(f"oracle step failed: {RC_NAMES.get(rc, rc)}")
        return out

    def step_no_reuse(self, topk, ctx_len, row_base, host_rows) -> StepOut:
        """The "KV Offload" comparison point (AVSG page, section 4.1): every
        valid selected id is copied, position i of token g to slot g*K + i.
        ctx_len is accepted for symmetry with step() and not used."""
        B, Nq, K = self.B, self.Nq, self.K
        topk = np.ascontiguousarray(topk, np.int32).reshape(B, Nq, K)
        row_base = np.ascontiguousarray(row_base, np.int64).reshape(B)
        host_rows = np.ascontiguousarray(host_rows, np.int32).reshape(B)
        out = StepOut(np.empty((B, Nq, K), np.int32), np.empty((B, Nq, K), np.int8),
                      np.empty((B, Nq), np.int32), np.zeros((B, Nq, K, 2), np.int32))
        hk = self.host_kv
        rc = _load().orc_step_no_reuse(ctypes.byref(self.cfg), _ptr(self.CNT), _ptr(topk),
                                       _ptr(row_base), _ptr(host_rows),
                                       _ptr(hk) if self.shadow is not None else None,
                                       _ptr(self.shadow), _ptr(out.slot_table),
                                       _ptr(out.hit_mask), _ptr(out.n_miss),
                                       _ptr(out.miss_pairs))
        if rc != 0:
            raise OracleError(f"oracle step failed: {RC_NAMES.get(rc, rc)}")
        return out

    def step_dense(self, topk, ctx_len, row_base, host_rows, map_len) -> StepOut:
        """AVSG slot management with an exact id -> slot map instead of the
        hash table (see orc_step_dense).  The map, int32 [B][map_len], lives
        in ``self.map`` (created on first use, all -1)."""
        B, Nq, K = self.B, self.Nq, self.K
        if getattr(self, "map", None) is None or self.map.shape != (B, map_len):
            self.map = np.full((B, map_len), -1, np.int32)
        topk = np.ascontiguousarray(topk, np.int32).reshape(B, Nq, K)
        ctx_len = np.ascontiguousarray(ctx_len, np.int32).reshape(B)
        row_base = np.ascontiguousarray(row_base, np.int64).reshape(B)
        host_rows = np.ascontiguousarray(host_rows, np.int32).reshape(B)
        out = StepOut(np.empty((B, Nq, K), np.int32), np.empty((B, Nq, K), np.int8),
                      np.empty((B, Nq), np.int32), np.zeros((B, Nq, K, 2), np.int32))
        hk = self.host_kv
        rc = _load().orc_step_dense(ctypes.byref(self.cfg), _ptr(self.C), _ptr(self.F),
                                    _ptr(self.CNT), _ptr(self.map), int(map_len),
                                    _ptr(topk), _ptr(ctx_len), _ptr(row_base),
                                    _ptr(host_rows),
                                    _ptr(hk) if self.shadow is not None else None,
                                    _ptr(self.shadow), _ptr(out.slot_table),
                                    _ptr(out.hit_mask), _ptr(out.n_miss),
                                    _ptr(out.miss_pairs))
        if rc != 0:
            raise OracleError(f"oracle step failed: {RC_NAMES.get(rc, rc)}")
        return out

    def step_sort_merge(self, topk, ctx_len, row_base, host_rows) -> StepOut:
        """The sort-merge matcher the page compares against (GatherSelection
        style exact reuse, no lifetimes): see orc_step_sort_merge.  Uses C
        and CNT; Q and F stay as they are."""
        B, Nq, K = self.B, self.Nq, self.K
        topk = np.ascontiguousarray(topk, np.int32).reshape(B, Nq, K)
        ctx_len = np.ascontiguousarray(ctx_len, np.int32).reshape(B)
        row_base = np.ascontiguousarray(row_base, np.int64).reshape(B)
        host_rows = np.ascontiguousarray(host_rows, np.int32).reshape(B)
        out = StepOut(np.empty((B, Nq, K), np.int32), np.empty((B, Nq, K), np.int8),
                      np.empty((B, Nq), np.int32), np.zeros((B, Nq, K, 2), np.int32))
        hk = self.host_kv
        rc = _load().orc_step_sort_merge(ctypes.byref(self.cfg), _ptr(self.C), _ptr(self.CNT),
                                         _ptr(topk), _ptr(ctx_len), _ptr(row_base),
                                         _ptr(host_rows),
                                         _ptr(hk) if self.shadow is not None else None,
                                         _ptr(self.shadow), _ptr(out.slot_table),
                                         _ptr(out.hit_mask), _ptr(out.n_miss),
                                         _ptr(out.miss_pairs))
        if rc != 0:
            raise OracleError(f"oracle step failed: {RC_NAMES.get(rc, rc)}")
        return out

    def prefetch_select(self, scores, ctx_len, theta, cap) -> np.ndarray:
        """Prefetch candidates (ECHO decode prefetch), int32 [B][K]: see
        orc_prefetch_select."""
        scores = np.ascontiguousarray(scores, np.float32).reshape(self.B, -1)
        ctx_len = np.ascontiguousarray(ctx_len, np.int32).reshape(self.B)
        theta = np.ascontiguousarray(theta, np.float32).reshape(self.B)
        cap = np.ascontiguousarray(cap, np.int32).reshape(self.B)
        out = np.empty((self.B, self.K), np.int32)
        _load().orc_prefetch_select(ctypes.byref(self.cfg), _ptr(scores), scores.shape[1],
                                    _ptr(ctx_len), _ptr(theta), _ptr(cap), _ptr(out))
        return out

    @staticmethod
    def ema_threshold(kth, theta, alpha) -> np.ndarray:
        """Next threshold per request (float32): see orc_ema_threshold."""
        kth = np.ascontiguousarray(kth, np.float32)
        out = np.ascontiguousarray(theta, np.float32).copy()
        _load().orc_ema_threshold(kth.size, _ptr(kth), _ptr(out), float(alpha))
        return out

    def probe_buckets(self, x: int) -> list:
        out = np.empty(self.R + 1, np.int32)
        _load().orc_probe_buckets(ctypes.byref(self.cfg), int(x), _ptr(out))
        return out.tolist()

    def word(self, x: int, slot: int) -> int:
        return int(_load().orc_word(ctypes.byref(self.cfg), int(x), int(slot)))

    def snapshot(self):
        return dict(Q=self.Q.copy(), C=self.C.copy(), F=self.F.copy(),
                    CNT=self.CNT.copy())
