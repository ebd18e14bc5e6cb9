"""The C-ABI library loads, exports what include/avsg.h declares, and its
host-only entry points behave as documented (no GPU needed)."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

import recall_step_amd as r

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                      "include", "avsg.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(avsg_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(r.lib, n), n
    assert set(names) == set(r.EXPORTED)


def test_version_and_strerror():
    assert r.avsg_version() == 1
    for code in (0, -1, -2, -3, -4, -5):
        assert r.avsg_strerror(code)
    assert "unknown" in r.avsg_strerror(-99)


def test_config_default_values():
    c = r.avsg_config_default(8, 1, 2048, 2048, 1280)
    assert (c.B, c.N_q, c.K, c.S, c.row_bytes) == (8, 1, 2048, 2048, 1280)
    assert (c.L, c.R, c.a1, c.a2, c.a_fp) == (15, 7, 0x9E3779B1, 0x85EBCA77, 0xC2B2AE3D)
    assert (c.flags, c.gather_blocks, c.stage1_threads) == (0, 0, 0)
    assert r.avsg_validate_config(c) == 0


@pytest.mark.parametrize("field,value", [
    ("S", 3000), ("S", 8), ("S", 131072), ("K", 0), ("K", 4096), ("B", 0),
    ("N_q", 0), ("L", 0), ("L", 128), ("R", -1), ("a1", 2), ("a2", 4),
    ("a_fp", 0), ("row_bytes", 1000), ("row_bytes", 0), ("flags", 64), ("flags", 6),
    ("flags", 24), ("flags", 40), ("flags", 48),
    ("gather_blocks", -1), ("stage1_threads", 128), ("stage1_threads", 300),
    ("stage1_threads", 2048)])
def test_invalid_configs_rejected(field, value):
    c = r.avsg_config_default(4, 1, 2048, 2048, 1280)
    setattr(c, field, value)
    assert r.avsg_validate_config(c) == r.AVSG_EINVAL


def test_probe_rounds_bounded_by_slots():
    """R <= S - 1: with an odd stride and S a power of two the probe sequence
    has visited every bucket after S rounds (AVSG s3.3, Probe primitive), so
    larger R is rejected instead of running rounds that only revisit."""
    c = r.avsg_config_default(1, 1, 16, 16, 1280)
    for R, rc in ((0, 0), (15, 0), (16, r.AVSG_EINVAL), (2**31 - 1, r.AVSG_EINVAL)):
        c.R = R
        assert r.avsg_validate_config(c) == rc, R
    c = r.avsg_config_default(1, 1, 2048, 8192, 1280)
    c.R = 8191
    assert r.avsg_validate_config(c) == 0
    c.R = 8192
    assert r.avsg_validate_config(c) == r.AVSG_EINVAL


def test_noalloc_step_rejects_a_miss_list_beyond_its_scratch():
    """avsg_step_noalloc keeps the miss list in a static array of
    AVSG_NOALLOC_MAX_PAIRS entries; a config needing more (with no
    caller-given miss list) is refused with AVSG_ESCRATCH before any HIP
    call or buffer access, so no GPU is needed here.  The pointers below
    are aligned placeholders that the call must never touch."""
    import ctypes
    K = 2048
    B = r.AVSG_NOALLOC_MAX_PAIRS // K + 1
    cfg = r.avsg_config_default(B, 1, K, 4096, 1280, flags=r.FLAG_SKIP_GATHER)
    fake = 1 << 20
    bufs = r.AvsgBuffers(fake, fake, fake, fake, fake, None, 1000, None, 0)
    io = r.AvsgStepIO(fake, fake, fake, fake, fake, fake, fake, None)
    rc = r.lib.avsg_step_noalloc(ctypes.byref(cfg), ctypes.byref(bufs), ctypes.byref(io),
                                 None)
    assert rc == r.AVSG_ESCRATCH
    assert "scratch" in r.avsg_strerror(rc)
    cfg.B = 0  # an invalid config is still EINVAL, checked first
    assert r.lib.avsg_step_noalloc(ctypes.byref(cfg), ctypes.byref(bufs), ctypes.byref(io),
                                   None) == r.AVSG_EINVAL


def test_capacity_bound_enforced():
    """N_q * K <= S (AVSG App. B slot preservation)."""
    assert r.avsg_validate_config(r.avsg_config_default(1, 4, 2048, 8192, 1280)) == 0
    assert r.avsg_validate_config(r.avsg_config_default(1, 4, 2049, 8192, 1280)) == r.AVSG_EINVAL


def test_lds_and_workspace_sizes():
    c = r.avsg_config_default(32, 1, 2048, 8192, 1280)
    # 9 bytes per slot (two int32 arrays + int8 lifetimes) + 4 B per victim +
    # a miss-rank bitmap over 2^18 ids with uint16 prefix counts per word
    # (6 B per 32 ids, larger than the 8 B per sort key of the fallback) +
    # 16 copies of the (L+2)-bin lifetime histogram + scratch.
    lds = r.avsg_stage1_lds_bytes(c)
    base = 9 * 8192 + 4 * 2048 + 6 * (1 << 18) // 32 + 16 * (15 + 2) * 4
    assert base <= lds <= base + 1024
    assert lds <= 160 * 1024
    assert r.avsg_workspace_bytes(c) == 32 * 1 * 2048 * 2 * 4
    # K = S = 8192 cannot be staged in 160 KiB: reported as 0 (unsupported).
    assert r.avsg_stage1_lds_bytes(r.avsg_config_default(1, 1, 8192, 8192, 1280)) == 0
    for K, S in [(1, 16), (256, 512), (2048, 2048), (4096, 8192), (256, 16384)]:
        lds = r.avsg_stage1_lds_bytes(r.avsg_config_default(1, 1, K, S, 1280))
        assert 9 * S + 4 * K + 8 * K <= lds <= 160 * 1024


def test_create_rejects_bad_arguments_before_touching_a_device():
    c = r.avsg_config_default(1, 1, 16, 16, 16)
    bufs = r.AvsgBuffers()
    with pytest.raises(r.AvsgError) as e:
        r.avsg_create(c, bufs)
    assert e.value.code == r.AVSG_EINVAL
    c.S = 24
    with pytest.raises(r.AvsgError) as e:
        r.avsg_create(c, r.AvsgBuffers(16, 16, 16, 16, 16, 16, 1))
    assert e.value.code == r.AVSG_EINVAL
    # misaligned state pointer
    c.S = 16
    with pytest.raises(r.AvsgError):
        r.avsg_create(c, r.AvsgBuffers(17, 32, 48, 64, 80, 96, 1))
    # the dense matcher needs its map (non-NULL, 4-byte aligned, map_len >= 1)
    c.flags = r.FLAG_DENSE_MAP
    for m, n in ((None, 100), (64, 0), (66, 100)):
        with pytest.raises(r.AvsgError) as e:
            r.avsg_create(c, r.AvsgBuffers(16, 32, 48, 64, 80, 96, 1, m, n))
        assert e.value.code == r.AVSG_EINVAL


def test_null_safe_destroy_and_free():
    assert r.lib.avsg_destroy(None) == 0
    assert r.lib.avsg_host_free(None) == 0
    assert r.lib.avsg_step(None, None, None) == r.AVSG_EINVAL
    assert r.lib.avsg_match(None, None, None) == r.AVSG_EINVAL
    assert r.lib.avsg_gather(None, None, None) == r.AVSG_EINVAL
    assert r.lib.avsg_state_init(None, None, None) == r.AVSG_EINVAL
    out = ctypes.c_void_p()
    assert r.lib.avsg_host_alloc(0, ctypes.byref(out)) == r.AVSG_EINVAL


def test_product_does_not_import_the_oracle():
    """The product path never routes through the oracle."""
    import recall_step_amd
    pkg = os.path.dirname(recall_step_amd.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".h")):
                text = open(os.path.join(root, f)).read()
                assert "oracle" not in text.lower(), f


def test_header_compiles_as_c99_and_links(tmp_path):
    """A plain C program includes the header, links the library and calls
    the entry points that need no GPU: the ABI is C, not C++."""
    import shutil
    import subprocess
    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    lib_dir = os.path.dirname(r._LIB_PATH)
    src = tmp_path / "use_avsg.c"
    src.write_text(r"""
#include <stdio.h>
#include "avsg.h"
int main(void) {
    avsg_config c;
    avsg_buffers bufs = {0};
    avsg_handle* h = (avsg_handle*)1;
    if (avsg_version() != AVSG_VERSION) return 1;
    avsg_config_default(&c, 8, 1, 2048, 2048, 1280);
    if (avsg_validate_config(&c) != AVSG_OK) return 2;
    if (avsg_stage1_lds_bytes(&c) == 0 || avsg_workspace_bytes(&c) != 8u * 2048u * 8u) return 3;
    c.R = c.S;
    if (avsg_validate_config(&c) != AVSG_EINVAL) return 7;
    c.R = 7;
    c.S = 3000;
    if (avsg_validate_config(&c) != AVSG_EINVAL) return 4;
    if (avsg_create(&c, &bufs, &h) != AVSG_EINVAL || h != NULL) return 5;
    if (avsg_destroy(NULL) != AVSG_OK) return 6;
    printf("%s\n", avsg_strerror(AVSG_EUNSUPPORTED));
    return 0;
}
""")
    exe = tmp_path / "use_avsg"
    cmd = [cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
           "-I", os.path.join(root, "include"), str(src), "-o", str(exe),
           "-L", lib_dir, "-lavsg", f"-Wl,-rpath,{lib_dir}"]
    b = subprocess.run(cmd, capture_output=True, text=True)
    assert b.returncode == 0, b.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert run.returncode == 0, (run.returncode, run.stderr)
    assert "beyond this build" in run.stdout
