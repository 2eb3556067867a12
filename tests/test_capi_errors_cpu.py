"""Argument checks of moe_cache_create that return before any HIP call (CPU)."""
import ctypes

import expert_offload_lru_amd as moe


def _create(*args):
    lib = moe.gpu_lib()
    h = ctypes.c_void_p()
    rc = lib.moe_cache_create(*args, ctypes.byref(h))
    return rc, h.value


def test_cache_smaller_than_top_k():
    rc, h = _create(128, 7, 8, 2048, 768, moe.Q_INT4_G32_F16, 48, 0)
    assert rc == moe.ERR_CACHE_TOO_SMALL and not h
    assert b"top_k" in moe.gpu_lib().moe_last_error()


def test_bad_arguments():
    assert _create(128, 92, 8, 2048, 768, 9, 48, 0)[0] == moe.ERR_INVALID          # unknown format
    assert _create(0, 92, 8, 2048, 768, 1, 48, 0)[0] == moe.ERR_INVALID
    assert _create(4, 92, 8, 2048, 768, 1, 48, 0)[0] == moe.ERR_INVALID            # top_k > E


def test_unsupported_shapes():
    assert _create(128, 92, 8, 2000, 768, 1, 48, 0)[0] == moe.ERR_UNSUPPORTED      # not a multiple of 256
    assert _create(128, 92, 8, 2048, 800, 2, 48, 0)[0] == moe.ERR_UNSUPPORTED
    assert _create(128, 92, 17, 2048, 768, 1, 48, 0)[0] == moe.ERR_UNSUPPORTED     # top_k > 16
    assert _create(2048, 92, 8, 2048, 768, 1, 48, 0)[0] == moe.ERR_UNSUPPORTED    # E > 1024


def test_null_cache_is_refused_by_the_opt_in_entry_points():
    """The captured-step and two-tier-store switches check their arguments before any HIP call."""
    lib = moe.gpu_lib()
    assert lib.moe_cache_set_graph(None, 1) == moe.ERR_INVALID
    assert lib.moe_cache_set_file_store(None, b"/nonexistent", 64, 4) == moe.ERR_INVALID
    assert lib.moe_cache_set_file_store(None, None, 64, 4) == moe.ERR_INVALID
