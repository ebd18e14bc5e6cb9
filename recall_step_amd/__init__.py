"""Python binding of the per-decode-step KV recall library (MI355X, gfx950).

Every step of the recall path runs in the HIP kernels of ``lib/libavsg.so``;
this package only marshals arguments into its C ABI (``include/avsg.h``).
The functions keep the C names and raise :class:`AvsgError` on a negative
return code.  :class:`RecallStep` and :class:`HostPool` bundle the buffers a
caller needs as torch device tensors and pinned host memory.

Importing fails loudly when the library has not been built: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
# torch ships its own HIP runtime with the same soname as ROCm's.  Loading it
# first makes the library below bind to that one copy; loading the library
# first would put two HIP runtimes in the process.
import torch  # noqa: F401

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lib", "libavsg.so")

if not os.path.exists(_LIB_PATH):
    raise ImportError(
        f"{_LIB_PATH} is missing: build the HIP library first "
        "(python recall_step_amd/build.py, or __graft_entry__.build())")

lib = ctypes.CDLL(_LIB_PATH)

AVSG_OK = 0
AVSG_EINVAL = -1
AVSG_ENOMEM = -2
AVSG_EHIP = -3
AVSG_EUNSUPPORTED = -4
AVSG_ESCRATCH = -5
# Miss-list entries the static scratch of avsg_step_noalloc holds per device.
AVSG_NOALLOC_MAX_PAIRS = 1 << 18

CNT_HITS, CNT_LOOKUPS, CNT_MISSES, CNT_LOST_COLLISION, CNT_LOST_EXHAUSTED, \
    CNT_LIVE_EVICTIONS, CNT_ERRORS, CNT_PROBE_VISITS = range(8)
ERR_OUT_OF_RANGE = 1
ERR_DUPLICATE = 2
FLAG_SKIP_GATHER = 1
FLAG_GATHER_BY_REQUEST = 2
FLAG_GATHER_BY_TOPK = 4
FLAG_NO_REUSE = 8
FLAG_SORT_MERGE = 16
FLAG_DENSE_MAP = 32


class AvsgConfig(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("N_q", ctypes.c_int32),
                ("K", ctypes.c_int32), ("S", ctypes.c_int32),
                ("L", ctypes.c_int32), ("R", ctypes.c_int32),
                ("a1", ctypes.c_uint32), ("a2", ctypes.c_uint32),
                ("a_fp", ctypes.c_uint32), ("row_bytes", ctypes.c_int32),
                ("flags", ctypes.c_uint32), ("gather_blocks", ctypes.c_int32),
                ("stage1_threads", ctypes.c_int32)]


class AvsgBuffers(ctypes.Structure):
    _fields_ = [("Q", ctypes.c_void_p), ("C", ctypes.c_void_p),
                ("F", ctypes.c_void_p), ("CNT", ctypes.c_void_p),
                ("dev_kv", ctypes.c_void_p), ("host_kv", ctypes.c_void_p),
                ("host_rows_total", ctypes.c_int64),
                ("map", ctypes.c_void_p), ("map_len", ctypes.c_int64)]


class AvsgStepIO(ctypes.Structure):
    _fields_ = [("topk", ctypes.c_void_p), ("ctx_len", ctypes.c_void_p),
                ("row_base", ctypes.c_void_p), ("host_rows", ctypes.c_void_p),
                ("slot_table", ctypes.c_void_p), ("hit_mask", ctypes.c_void_p),
                ("n_miss", ctypes.c_void_p), ("miss_pairs", ctypes.c_void_p)]


_p = ctypes.c_void_p
_sigs = {
    "avsg_version": ([], ctypes.c_int),
    "avsg_strerror": ([ctypes.c_int], ctypes.c_char_p),
    "avsg_last_hip_error": ([], ctypes.c_int),
    "avsg_config_default": ([ctypes.POINTER(AvsgConfig), ctypes.c_int32, ctypes.c_int32,
                             ctypes.c_int32, ctypes.c_int32, ctypes.c_int32], None),
    "avsg_validate_config": ([ctypes.POINTER(AvsgConfig)], ctypes.c_int),
    "avsg_stage1_lds_bytes": ([ctypes.POINTER(AvsgConfig)], ctypes.c_size_t),
    "avsg_workspace_bytes": ([ctypes.POINTER(AvsgConfig)], ctypes.c_size_t),
    "avsg_create": ([ctypes.POINTER(AvsgConfig), ctypes.POINTER(AvsgBuffers),
                     ctypes.POINTER(_p)], ctypes.c_int),
    "avsg_destroy": ([_p], ctypes.c_int),
    "avsg_state_init": ([_p, _p, _p], ctypes.c_int),
    "avsg_match": ([_p, ctypes.POINTER(AvsgStepIO), _p], ctypes.c_int),
    "avsg_gather": ([_p, ctypes.POINTER(AvsgStepIO), _p], ctypes.c_int),
    "avsg_step": ([_p, ctypes.POINTER(AvsgStepIO), _p], ctypes.c_int),
    "avsg_match_continue": ([_p, ctypes.POINTER(AvsgStepIO), _p], ctypes.c_int),
    "avsg_step_noalloc": ([ctypes.POINTER(AvsgConfig), ctypes.POINTER(AvsgBuffers),
                           ctypes.POINTER(AvsgStepIO), _p], ctypes.c_int),
    "avsg_prefetch_select": ([_p, _p, ctypes.c_int64, _p, _p, _p, _p, _p], ctypes.c_int),
    "avsg_ema_threshold": ([_p, _p, _p, ctypes.c_float, _p], ctypes.c_int),
    "avsg_host_alloc": ([ctypes.c_size_t, ctypes.POINTER(_p)], ctypes.c_int),
    "avsg_host_free": ([_p], ctypes.c_int),
}
for _name, (_args, _res) in _sigs.items():
    _f = getattr(lib, _name)
    _f.argtypes = _args
    _f.restype = _res

EXPORTED = tuple(_sigs)


class AvsgError(RuntimeError):
    def __init__(self, code: int, what: str):
        msg = f"{what}: {avsg_strerror(code)} ({code})"
        if code == AVSG_EHIP:
            msg += f", hipError {lib.avsg_last_hip_error()}"
        super().__init__(msg)
        self.code = code


def _check(code: int, what: str) -> int:
    if code < 0:
        raise AvsgError(code, what)
    return code


# ------------------------------------------------ C functions, same names --

def avsg_version() -> int:
    return lib.avsg_version()


def avsg_strerror(code: int) -> str:
    return lib.avsg_strerror(code).decode()


def avsg_config_default(B, N_q, K, S, row_bytes, **overrides) -> AvsgConfig:
    cfg = AvsgConfig()
    lib.avsg_config_default(ctypes.byref(cfg), B, N_q, K, S, row_bytes)
    for k, v in overrides.items():
        setattr(cfg, k, v)
    return cfg


def avsg_validate_config(cfg: AvsgConfig) -> int:
    return lib.avsg_validate_config(ctypes.byref(cfg))


def avsg_stage1_lds_bytes(cfg: AvsgConfig) -> int:
    return lib.avsg_stage1_lds_bytes(ctypes.byref(cfg))


def avsg_workspace_bytes(cfg: AvsgConfig) -> int:
    return lib.avsg_workspace_bytes(ctypes.byref(cfg))


def avsg_create(cfg: AvsgConfig, bufs: AvsgBuffers) -> int:
    h = _p()
    _check(lib.avsg_create(ctypes.byref(cfg), ctypes.byref(bufs), ctypes.byref(h)),
           "avsg_create")
    return h.value


def avsg_destroy(h) -> None:
    _check(lib.avsg_destroy(h), "avsg_destroy")


def avsg_state_init(h, row_mask_ptr, stream) -> None:
    _check(lib.avsg_state_init(h, row_mask_ptr, stream), "avsg_state_init")


def avsg_match(h, io: AvsgStepIO, stream) -> None:
    _check(lib.avsg_match(h, ctypes.byref(io), stream), "avsg_match")


def avsg_gather(h, io: AvsgStepIO, stream) -> None:
    _check(lib.avsg_gather(h, ctypes.byref(io), stream), "avsg_gather")


def avsg_step(h, io: AvsgStepIO, stream) -> None:
    _check(lib.avsg_step(h, ctypes.byref(io), stream), "avsg_step")


def avsg_match_continue(h, io: AvsgStepIO, stream) -> None:
    _check(lib.avsg_match_continue(h, ctypes.byref(io), stream), "avsg_match_continue")


def avsg_step_noalloc(cfg: AvsgConfig, bufs: AvsgBuffers, io: AvsgStepIO, stream) -> None:
    _check(lib.avsg_step_noalloc(ctypes.byref(cfg), ctypes.byref(bufs), ctypes.byref(io),
                                 stream), "avsg_step_noalloc")


def avsg_prefetch_select(h, scores_ptr, row_len, ctx_len_ptr, theta_ptr, cap_ptr, cand_ptr,
                         stream) -> None:
    _check(lib.avsg_prefetch_select(h, scores_ptr, int(row_len), ctx_len_ptr, theta_ptr,
                                    cap_ptr, cand_ptr, stream), "avsg_prefetch_select")


def avsg_ema_threshold(h, kth_ptr, theta_ptr, alpha, stream) -> None:
    _check(lib.avsg_ema_threshold(h, kth_ptr, theta_ptr, float(alpha), stream),
           "avsg_ema_threshold")


def avsg_host_alloc(nbytes: int) -> int:
    out = _p()
    _check(lib.avsg_host_alloc(nbytes, ctypes.byref(out)), "avsg_host_alloc")
    return out.value


def avsg_host_free(ptr) -> None:
    _check(lib.avsg_host_free(ptr), "avsg_host_free")


# ------------------------------------------------------------ conveniences --

class HostPool:
    """Pinned, device-mapped host bytes from ``avsg_host_alloc``.

    ``array`` is a numpy uint8 view of the whole pool (for filling it)."""

    def __init__(self, nbytes: int):
        self.nbytes = int(nbytes)
        self.ptr = avsg_host_alloc(max(self.nbytes, 16))
        buf = (ctypes.c_uint8 * self.nbytes).from_address(self.ptr)
        self.array = np.frombuffer(buf, dtype=np.uint8)

    def close(self):
        if self.ptr:
            self.array = None
            avsg_host_free(self.ptr)
            self.ptr = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def _dptr(t):
    return None if t is None else t.data_ptr()


def _stream_handle(stream):
    import torch
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


class RecallStep:
    """Caller-side buffers for one handle: state, slot buffer and outputs as
    torch device tensors on the current device, plus the handle itself."""

    def __init__(self, cfg: AvsgConfig, host: HostPool | None, host_rows_total: int,
                 stream=None, map_len: int = 0):
        import torch
        dev = torch.device("cuda", torch.cuda.current_device())
        B, Nq, K, S = cfg.B, cfg.N_q, cfg.K, cfg.S
        self.cfg = cfg
        self.host = host
        self.Q = torch.empty((B, S), dtype=torch.int32, device=dev)
        self.C = torch.empty((B, S), dtype=torch.int32, device=dev)
        self.F = torch.empty((B, S), dtype=torch.int32, device=dev)
        self.CNT = torch.empty((B, 8), dtype=torch.int32, device=dev)
        # Without the copy stage the slot buffer is never touched.
        kv_shape = (1, 1, 16) if cfg.flags & FLAG_SKIP_GATHER else (B, S, cfg.row_bytes)
        self.dev_kv = torch.zeros(kv_shape, dtype=torch.uint8, device=dev)
        self.slot_table = torch.empty((B, Nq, K), dtype=torch.int32, device=dev)
        self.hit_mask = torch.empty((B, Nq, K), dtype=torch.int8, device=dev)
        self.n_miss = torch.empty((B, Nq), dtype=torch.int32, device=dev)
        self.miss_pairs = torch.zeros((B, Nq, K, 2), dtype=torch.int32, device=dev)
        # The dense matcher's id -> slot map, one row of map_len ids per request.
        self.map = (torch.empty((B, map_len), dtype=torch.int32, device=dev)
                    if cfg.flags & FLAG_DENSE_MAP else None)
        self.bufs = AvsgBuffers(_dptr(self.Q), _dptr(self.C), _dptr(self.F),
                                _dptr(self.CNT), _dptr(self.dev_kv),
                                host.ptr if host is not None else None,
                                int(host_rows_total), _dptr(self.map),
                                int(map_len) if self.map is not None else 0)
        self.handle = avsg_create(cfg, self.bufs)
        self.state_init(stream=stream)

    def state_init(self, row_mask=None, stream=None):
        avsg_state_init(self.handle, _dptr(row_mask), _stream_handle(stream))

    def io(self, topk, ctx_len, row_base, host_rows, miss_pairs=True) -> AvsgStepIO:
        """Step io over device tensors (topk int32 [B][N_q][K], ctx_len int32
        [B], row_base int64 [B], host_rows int32 [B]) and this object's
        outputs.  ``miss_pairs=False`` leaves the miss list in the library's
        workspace."""
        return AvsgStepIO(_dptr(topk), _dptr(ctx_len), _dptr(row_base), _dptr(host_rows),
                          _dptr(self.slot_table), _dptr(self.hit_mask),
                          _dptr(self.n_miss),
                          _dptr(self.miss_pairs) if miss_pairs else None)

    def step(self, io: AvsgStepIO, stream=None):
        avsg_step(self.handle, io, _stream_handle(stream))

    def match(self, io: AvsgStepIO, stream=None):
        avsg_match(self.handle, io, _stream_handle(stream))

    def match_continue(self, io: AvsgStepIO, stream=None):
        avsg_match_continue(self.handle, io, _stream_handle(stream))

    def gather(self, io: AvsgStepIO, stream=None):
        avsg_gather(self.handle, io, _stream_handle(stream))

    def close(self):
        if self.handle:
            avsg_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
