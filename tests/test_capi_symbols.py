"""The C-ABI libraries load on a CPU-only machine and export every function the
headers declare (no compute calls)."""
import ctypes
import os
import re
import subprocess

import pytest

import expert_offload_lru_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared(header):
    with open(os.path.join(ROOT, "include", header)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", text)) - {"moe_trace_fn"})


def _exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], stdout=subprocess.PIPE, text=True, check=True).stdout
    return {l.split()[-1] for l in out.splitlines() if " T " in l}


def test_headers_declare_the_core_entry_points():
    decl = _declared("moe_offload.h")
    for name in ("moe_cache_create", "moe_layer_forward", "moe_cache_stats", "moe_cache_destroy"):
        assert name in decl


@pytest.mark.parametrize("header", ["moe_offload.h", "moe_planner.h"])
def test_gpu_library_exports_every_declared_function(header):
    exported = _exported(moe.LIB_PATH)
    missing = [n for n in _declared(header) if n not in exported]
    assert not missing, missing


def test_planner_library_exports_planner_functions():
    exported = _exported(moe.PLANNER_LIB_PATH)
    missing = [n for n in _declared("moe_planner.h") if n not in exported]
    assert not missing, missing


def test_gpu_library_loads_without_a_gpu():
    lib = moe.gpu_lib()
    assert lib.moe_expert_bytes(moe.Q_INT4_G32_F16, 2048, 768) == 2654208
    assert lib.moe_expert_bytes(moe.Q_E2M1_E4M3_G16, 3072, 512) == 2654208
    assert lib.moe_expert_bytes(moe.Q_F32, 256, 128) == 393216
    assert lib.moe_expert_bytes(7, 256, 128) == 0
    assert isinstance(lib.moe_last_error(), bytes)


def test_no_cpu_fallback_in_the_library_sources():
    # the product never imports the oracle
    pkg = os.path.join(ROOT, "expert_offload_lru_amd")
    for dirpath, _dirs, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".cpp", ".hip", ".hpp")):
                with open(os.path.join(dirpath, f)) as fh:
                    src = fh.read()
                assert "import oracle" not in src and "from oracle" not in src, f
