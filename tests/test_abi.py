"""CPU-side checks of the C-ABI library: it loads, exports every symbol the
header declares, and its host-only paths (status strings, argument
validation that fails before any device call) behave as documented."""
import ctypes
import os
import re

import pytest

import sparse_attention_hop_amd as sah

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "diffuser.h")


def header_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"DIFFUSER_API\s+[\w\s\*]*?\b(diffuser_\w+)\s*\(", text)))


def test_header_lists_binding_symbols():
    assert header_symbols() == sorted(sah.ABI_SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = sah.load_library()
    for name in header_symbols():
        assert hasattr(lib, name), name


def test_only_abi_symbols_exported():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", sah.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = sorted(line.split()[-1] for line in out.splitlines() if " T " in line)
    assert exported == header_symbols()


def test_status_strings():
    lib = sah.load_library()
    for code, name in sah.STATUS_NAMES.items():
        assert lib.diffuser_status_string(code).decode() == name


def test_build_graph_rejects_bad_descriptors_on_host():
    lib = sah.load_library()
    out = ctypes.c_void_p()
    bad = [
        sah._GraphDesc(0, 1, 0, None, 0, 1, 0, 0),          # n < 1
        sah._GraphDesc(10, -1, 0, None, 0, 1, 0, 0),        # r < 0
        sah._GraphDesc(10, 1, 1, None, 0, 1, 0, 0),         # NULL globals
        sah._GraphDesc(10, 1, 0, None, -3, 1, 0, 0),        # R < 0
        sah._GraphDesc(10, 1, 0, None, 0, 0, 0, 0),         # num_graphs < 1
        sah._GraphDesc(10, 1, 0, None, 0, 1, 2, 0),         # causal not 0/1
    ]
    for d in bad:
        assert lib.diffuser_build_graph(ctypes.byref(d), None, ctypes.byref(out)) == 1
        assert lib.diffuser_last_error().decode()
        assert out.value is None
    g = (ctypes.c_int32 * 2)(5, 5)
    d = sah._GraphDesc(10, 1, 2, ctypes.cast(g, ctypes.c_void_p), 0, 1, 0, 0)
    assert lib.diffuser_build_graph(ctypes.byref(d), None, ctypes.byref(out)) == 1
    # a sampled random budget above 1024 is unsupported
    d = sah._GraphDesc(5000, 1, 0, None, 2000, 1, 0, 0)
    assert lib.diffuser_build_graph(ctypes.byref(d), None, ctypes.byref(out)) == 2


def test_null_handles_rejected_on_host():
    lib = sah.load_library()
    size = ctypes.c_size_t()
    assert lib.diffuser_attn_workspace_size(None, 1, 1, 64, 64, 0, ctypes.byref(size)) == 1
    assert lib.diffuser_diffuse_workspace_size(None, 1, 1, 64, 3, 0, ctypes.byref(size)) == 1
    assert lib.diffuser_graph_info(None, None, None, None, None) == 1
    lib.diffuser_graph_destroy(None)
    assert lib.diffuser_attn(None, None, None, 0, 1, 1, 64, 64, None, 1, 0.1, None, None, 0,
                             None) == 1
    assert lib.diffuser_csr_workspace_size(None, 1, 1, 64, 3, 0, ctypes.byref(size)) == 1
    assert lib.diffuser_scores_softmax_csr(None, None, 0, 1, 1, 64, None, None, None, 0,
                                           None) == 1
    assert lib.diffuser_diffuse_csr(None, None, 0, 1, 1, 64, None, 3, 0.1, None, None, 0,
                                    None) == 1


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError, match="missing"):
        sah.load_library(str(tmp_path / "nope.so"))
