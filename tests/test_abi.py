"""The C-ABI library loads and exports every function include/pa.h declares (no GPU)."""
import ctypes
import os
import re

import pytest

from conftest import ROOT

HEADER = os.path.join(ROOT, "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("pa_cache_write", "pa_decode", "pa_copy_blocks", "pa_decode_workspace_size",
                 "pa_status_string", "pa_bm_create", "pa_bm_append_slot"):
        assert must in names


def test_library_exports_every_declared_symbol():
    import paged_kv_cache_write_amd as pk
    lib = pk.lib()
    raw = ctypes.CDLL(pk.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, missing
    assert lib.pa_version() >= 100


def test_debug_library_exports_the_same_symbols():
    """libpa_debug.so (PA_DEBUG: device checks of slots, block ids and copy pairs)
    exports the same ABI and says it is the debug build; libpa.so says it is not."""
    import paged_kv_cache_write_amd as pk
    raw = ctypes.CDLL(pk.LIB_DEBUG_PATH)
    missing = [n for n in declared_functions() if not hasattr(raw, n)]
    assert not missing, missing
    assert pk.lib().pa_debug_enabled() == 0
    prev = pk.use_debug_library(True)
    try:
        assert pk.lib().pa_debug_enabled() == 1
    finally:
        pk.use_debug_library(prev)
    assert pk.lib().pa_debug_enabled() == 0


def test_status_strings():
    import paged_kv_cache_write_amd as pk
    lib = pk.lib()
    for code in range(0, -9, -1):
        s = lib.pa_status_string(code).decode()
        assert s.startswith("PA_")
    assert lib.pa_status_string(-99) == b"unknown pa status"


def test_host_side_argument_checks_enqueue_nothing():
    """Invalid shapes fail on the host, before any device work (safe without a GPU)."""
    import paged_kv_cache_write_amd as pk
    lib = pk.lib()
    # unsupported head_dim / block size / dtype
    assert lib.pa_cache_write(None, None, None, 1, None, None, 1, 1, 96, 16, 1, None) == -2
    assert lib.pa_cache_write(None, None, None, 1, None, None, 1, 1, 128, 12, 1, None) == -2
    assert lib.pa_cache_write(None, None, None, 1, None, None, 1, 1, 128, 16, 7, None) == -2
    # null pointers
    assert lib.pa_cache_write(None, None, None, 1, None, None, 1, 1, 128, 16, 1, None) == -1
    # zero tokens is a no-op even with null pointers
    assert lib.pa_cache_write(None, None, None, 0, None, None, 1, 1, 128, 16, 1, None) == 0
    assert lib.pa_copy_blocks(None, None, None, 0, 1, 1, 128, 16, 1, None) == 0
    # decode: zero sequences is a no-op; missing workspace for a split plan
    args = [None, None, None, None, 1, None, 0, 40, 128, 16, 4096, 0.1, 2048, 1, None, None, 0, 0,
            None]
    assert lib.pa_decode(*args) == 0
    args[6] = 30
    args[0] = args[1] = args[2] = args[3] = args[5] = args[14] = 256   # fake aligned pointers
    assert lib.pa_decode(*args) == -5          # split plan, no workspace: rejected on the host
    args[17] = 48                              # partition not a multiple of 32
    assert lib.pa_decode(*args) == -1
    # streaming read: zero bytes is a no-op; sizes must be whole 8 KiB chunks
    assert lib.pa_stream_read(None, 0, None, 0, None) == 0
    assert lib.pa_stream_read(256, 8192 + 16, 512, 0, None) == -1
    assert lib.pa_stream_read(None, 8192, 512, 0, None) == -1
    assert lib.pa_stream_read(264, 8192, 512, 0, None) == -1     # src not 16-byte aligned
    # gathered tile read: no units is a no-op; tiles are powers of two from 1 KiB to 1 MiB
    assert lib.pa_tile_read(None, None, 4096, 0, None, None, 0, None, None) == 0
    assert lib.pa_tile_read(256, 512, 3072, 8, 768, 1024, 1, 1280, None) == -1   # not a power of 2
    assert lib.pa_tile_read(256, 512, 512, 8, 768, 1024, 1, 1280, None) == -1    # below 1 KiB
    assert lib.pa_tile_read(256, 512, 2 << 20, 8, 768, 1024, 1, 1280, None) == -1  # above 1 MiB
    assert lib.pa_tile_read(264, 512, 4096, 8, 768, 1024, 1, 1280, None) == -1   # a not aligned
    assert lib.pa_tile_read(256, 512, 4096, 8, None, 1024, 1, 1280, None) == -1  # no offsets
    assert lib.pa_tile_read(256, 512, 4096, -1, 768, 1024, 1, 1280, None) == -1  # negative extent
    assert lib.pa_tile_read(256, 512, 4096, 8, 768, 1024, -1, 1280, None) == -1  # negative units


@pytest.mark.parametrize("S,H,D,bs,L,req", [(30, 40, 128, 16, 2048, 0), (8, 40, 128, 16, 4096, 512),
                                            (4, 4, 64, 16, 100, 0), (256, 40, 128, 8, 4096, 0),
                                            (256, 40, 128, 128, 4096, 0)])
def test_decode_plan(S, H, D, bs, L, req):
    import paged_kv_cache_write_amd as pk
    pt, parts, ws = pk.decode_plan(S, H, D, bs, L, 1, req)
    assert pt % bs == 0 and pt % 32 == 0 and pt <= 64 * bs
    if req:
        assert pt == req
    assert parts == -(-L // pt)
    counters = -(-(S * H * 4) // 256) * 256           # one int32 per row, padded to 256 B
    ml = -(-(S * H * parts * 2) // 4) * 4                # (max, sum) floats, padded to 16 B
    assert ws == (0 if parts == 1 else counters + (ml + S * H * parts * D) * 4)
    assert pk.decode_workspace_size(S, H, D, bs, L, 1, req) == ws


def test_engine_staging_and_errors():
    import paged_kv_cache_write_amd as pk
    lib = pk.lib()
    assert lib.pa_engine_staging_bytes(30, 140, 16) > 30 * 140 * 4
    assert lib.pa_engine_staging_bytes(0, 140, 16) == 0
    import ctypes
    h = ctypes.c_void_p()
    assert lib.pa_engine_create(None, None, None, 1, 1, 128, 16, 1, 1, 1, 0, None, 1, None,
                                ctypes.byref(h)) == -1


def test_engine_rejects_batches_the_launches_cannot_hold():
    """More than 65535 sequences per step cannot be launched: pa_engine_create says
    so up front (no GPU call is made before that check), so no step can fail after
    its appends for that reason."""
    import ctypes
    import paged_kv_cache_write_amd as pk
    lib = pk.lib()
    bm = ctypes.c_void_p()
    assert lib.pa_bm_create(64, 16, None, 0, ctypes.byref(bm)) == 0
    try:
        h = ctypes.c_void_p()
        fake = 256                                     # aligned stand-ins, never dereferenced
        assert lib.pa_engine_create(bm, fake, fake, 64, 4, 128, 16, 1, 65536, 4, 0, fake, 2,
                                    fake, ctypes.byref(h)) == -2
        assert not h.value
    finally:
        lib.pa_bm_destroy(bm)
