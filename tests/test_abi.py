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


def test_cache_entry_points_reject_bad_arguments():
    import rejection_sampling_verify_spec_amd.specverify as b
    d = 256
    ok = (d, d + 4096, d, d + 8192, d + 16384, d + 20480, d + 24576)  # kc vc kn vn len nacc out
    assert b.spec_kv_commit(*ok, -1, 5, 4, 256, 4, 60, None) == b.SV_EINVAL          # B < 0
    assert b.spec_kv_commit(None, None, None, None, None, None, None, 0, 5, 4, 256, 4, 60, None) == b.SV_OK
    assert b.spec_kv_commit(*ok, 2, 5, 4, 256, 4, 0, None) == b.SV_EINVAL            # W = 0
    assert b.spec_kv_commit(*ok, 2, 5, 4, 256, -1, 8, None) == b.SV_EINVAL           # S < 0
    assert b.spec_kv_commit(*ok, 2, 5, 0, 256, 4, 8, None) == b.SV_EINVAL            # no rows
    assert b.spec_kv_commit(*ok, 2, 5, 4, 0, 4, 8, None) == b.SV_EINVAL              # empty rows
    assert b.spec_kv_commit(*ok, 2, 257, 4, 256, 4, 8, None) == b.SV_EINVAL          # gamma too large
    assert b.spec_kv_commit(*ok, 2, 5, 4, 256, 1 << 29, (1 << 29) + 1, None) == b.SV_EINVAL  # S + W too large
    assert b.spec_kv_commit(d, d, *ok[2:], 2, 5, 4, 256, 4, 8, None) == b.SV_EINVAL  # k_cache == v_cache
    bad = list(ok)
    bad[6] = ok[4] + 4  # new_lengths overlaps lengths
    assert b.spec_kv_commit(*bad, 2, 5, 4, 256, 4, 8, None) == b.SV_EINVAL
    bad[6] = None
    assert b.spec_kv_commit(*bad, 2, 5, 4, 256, 4, 8, None) == b.SV_EINVAL
    assert b.spec_kv_valid_slots(d, 2, 4, 0, d, None, d, None) == b.SV_EINVAL
    assert b.spec_kv_valid_slots(d, 2, 4, 8, None, None, d, None) == b.SV_EINVAL
    assert b.spec_kv_valid_slots(None, 0, 4, 8, None, None, None, None) == b.SV_OK
    # draft window: block bound, K above W, zero block size, short clone width
    assert b.spec_draft_window_max_blocks(64, 16) == 5 and b.spec_draft_window_max_blocks(63, 16) == 5
    assert b.spec_draft_window_max_blocks(2048, 128) == 17 and b.spec_draft_window_max_blocks(0, 16) == -1
    args = dict(seq=d, B=4, W=64, b=16, K=3, table=d + 64, cols=20, out=d + 4096, win=d + 8192, wc=5)

    def call(**kw):
        a = {**args, **kw}
        return b.spec_draft_window(a["seq"], a["B"], a["W"], a["b"], a["K"], a["table"], a["cols"], a["out"],
                                   a["win"], a["wc"], None)
    assert call(wc=4) == b.SV_EINVAL
    assert call(K=65) == b.SV_EINVAL
    assert call(b=0, wc=100) == b.SV_EINVAL
    assert call(B=-1) == b.SV_EINVAL
    assert call(B=0) == b.SV_OK
    assert call(table=None) == b.SV_EINVAL
    assert call(out=d + 4) == b.SV_EINVAL  # overlaps seq_lens without being it


def test_draft_window_host_matches_oracle():
    """The host-side windowed length (for host copies of the length inputs) runs here without a GPU."""
    import numpy as np

    import oracle
    import rejection_sampling_verify_spec_amd.specverify as b
    rng = np.random.default_rng(12)
    for W, bs, K in [(64, 16, 3), (63, 16, 0), (2048, 128, 5), (7, 3, 7), (1, 1, 0), (100, 7, 50)]:
        seq = np.concatenate([np.arange(-3, 4 * W + 3 * bs), rng.integers(0, 2 ** 31 - 1, 200),
                              [2 ** 31 - 1, -(2 ** 31)]]).astype(np.int32)
        out = np.empty_like(seq)
        assert b.spec_draft_window_host(seq.ctypes.data, seq.size, W, bs, K, out.ctypes.data) == b.SV_OK
        ref = [(-1 if oracle.window_one(int(L), W, bs, K) is None else oracle.window_one(int(L), W, bs, K)[1])
               for L in seq]
        assert out.tolist() == ref
        # in place
        assert b.spec_draft_window_host(seq.ctypes.data, seq.size, W, bs, K, seq.ctypes.data) == b.SV_OK
        assert seq.tolist() == ref
    assert b.spec_draft_window_host(None, 0, 64, 16, 3, None) == b.SV_OK
    assert b.spec_draft_window_host(None, 3, 64, 16, 3, None) == b.SV_EINVAL


def test_read_probe_rejects_bad_arguments():
    import rejection_sampling_verify_spec_amd.specverify as b
    assert b.spec_read_probe_words(0) == 0 and b.spec_read_probe_words(16) == 4
    assert b.spec_read_probe_words(2048 * 16 + 16) == 8
    assert b.spec_read_probe(256, 24, 512, None) == b.SV_EINVAL   # not a multiple of 16
    assert b.spec_read_probe(None, 32, 512, None) == b.SV_EINVAL
    assert b.spec_read_probe(264, 32, 512, None) == b.SV_EALIGN
    assert b.spec_read_probe(None, 0, None, None) == b.SV_OK
