"""The C-ABI library without a GPU: it loads, exports every function that
include/specverify.h declares, and rejects bad arguments on the host before
any HIP call (no compute is launched here)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "specverify.h")
LIB = os.path.join(ROOT, "rejection_sampling_verify_spec_amd", "libspecverify.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from rejection_sampling_verify_spec_amd import build
        build.build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(spec_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 12
    for n in names:
        assert hasattr(lib, n), n


def test_python_binding_names_match_header():
    import rejection_sampling_verify_spec_amd.specverify as b
    for n in declared_functions():
        assert callable(getattr(b, n)), n


def test_workspace_sizes(lib):
    f = lib.spec_verify_workspace_bytes
    f.restype = ctypes.c_size_t
    assert f(256, 5, 128256, 1) > 0
    assert f(256, 5, 128256, 1) % 256 == 0
    assert f(-1, 5, 100, 1) == 0 and f(4, -1, 100, 1) == 0 and f(4, 5, 0, 1) == 0 and f(4, 5, 100, 7) == 0
    assert f(512, 5, 128256, 1) > f(256, 5, 128256, 1)
    g = lib.spec_verify_tree_workspace_bytes
    g.restype = ctypes.c_size_t
    assert g(32, 64, 152064, 1) > 0 and g(32, 0, 100, 1) == 0 and g(32, 1025, 100, 1) == 0
    h = lib.spec_verify_ragged_workspace_bytes
    h.restype = ctypes.c_size_t
    assert h(1024, 4608, 8, 151936, 1) > 0 and h(4, -1, 8, 10, 1) == 0


def test_host_validation_errors(lib):
    import rejection_sampling_verify_spec_amd.specverify as b
    dummy = 256  # a non-null, aligned fake address; the calls below return before any use
    # B < 0, gamma out of range
    assert b.spec_verify(dummy, dummy, 1, dummy, dummy, dummy, dummy, -1, 5, 10, dummy, dummy, None, dummy, 1 << 20,
                         None) == b.SV_EINVAL
    assert b.spec_verify(dummy, dummy, 1, dummy, dummy, dummy, dummy, 2, 1025, 10, dummy, dummy, None, dummy,
                         1 << 20, None) == b.SV_EINVAL
    # B == 0 is a no-op
    assert b.spec_verify(None, None, 1, None, None, None, None, 0, 5, 10, None, None, None, None, 0, None) == b.SV_OK
    # bad dtype, null pointers, misaligned logits, short workspace
    assert b.spec_verify(dummy, dummy, 3, dummy, dummy, dummy, dummy, 2, 5, 10, dummy, dummy, None, dummy, 1 << 20,
                         None) == b.SV_EDTYPE
    assert b.spec_verify(None, dummy, 1, dummy, dummy, dummy, dummy, 2, 5, 10, dummy, dummy, None, dummy, 1 << 20,
                         None) == b.SV_EINVAL
    assert b.spec_verify(dummy + 1, dummy, 1, dummy, dummy, dummy, dummy, 2, 5, 10, dummy, dummy, None, dummy,
                         1 << 20, None) == b.SV_EALIGN
    assert b.spec_verify(dummy + 2, dummy, 0, dummy, dummy, dummy, dummy, 2, 5, 10, dummy, dummy, None, dummy,
                         1 << 20, None) == b.SV_EALIGN
    assert b.spec_verify(dummy, dummy, 1, dummy, dummy, dummy, dummy, 2, 5, 10, dummy, dummy, None, dummy, 16,
                         None) == b.SV_ENOWS
    assert b.spec_verify(dummy, dummy, 1, dummy, dummy, dummy, dummy, 2, 5, 10, dummy, dummy, None, dummy + 8,
                         1 << 20, None) == b.SV_ENOWS
    assert b.spec_verify(dummy, dummy, 1, dummy, dummy, dummy, dummy, 2, 5, 0, dummy, dummy, None, dummy, 1 << 20,
                         None) == b.SV_EINVAL
    # tree: N out of range, max_depth >= N
    assert b.spec_verify_tree(dummy, dummy, 1, dummy, dummy, dummy, dummy, dummy, 2, 0, 10, 0, dummy, dummy, dummy,
                              dummy, 1 << 20, None) == b.SV_EINVAL
    assert b.spec_verify_tree(dummy, dummy, 1, dummy, dummy, dummy, dummy, dummy, 2, 4, 10, 4, dummy, dummy, dummy,
                              dummy, 1 << 20, None) == b.SV_EINVAL
    # ragged: total_draft above B * gamma_max
    assert b.spec_verify_ragged(dummy, dummy, 1, dummy, 100, dummy, dummy, dummy, dummy, 4, 8, 10, dummy, dummy, None,
                                dummy, 1 << 20, None) == b.SV_EINVAL
    for code in (0, -1, -2, -3, -4, -5, -99):
        assert isinstance(b.spec_verify_strerror(code), str)
    assert b.spec_verify_version() == 1
