"""GPU parity of the draft-token sampler (spec_sample_rows through the C ABI)
against the oracle's sampler on the same seeded rows and uniforms.

Bar (as for the verify draw, tests/_parity.py): tokens equal the oracle's bit
for bit; a row may differ only when the oracle flags it as a near-tie (u*S
within 1e-5*S of a CDF boundary), and such rows must stay below 1e-4 of all
rows (zero for the sizes here).
"""
import numpy as np
import pytest

import inputgen
import oracle
from _parity import FLAG, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import torch

    import rejection_sampling_verify_spec_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


def check(sv, logits, T, u, label):
    import torch
    V = logits.shape[-1]
    logits = np.ascontiguousarray(logits.reshape(-1, V))
    rows = logits.shape[0]
    T = np.ascontiguousarray(np.broadcast_to(np.asarray(T, np.float32), (rows,)))
    u = np.ascontiguousarray(np.broadcast_to(np.asarray(u, np.float32), (rows,)))
    print(f"[{label}] rows {rows} V {V} {logits.dtype}", flush=True)
    out = sv.sample_rows(to_dev(logits), to_dev(T), to_dev(u))
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    ref = oracle.sample_rows(logits, T, u)
    mism = got != ref["tokens"]
    flagged = ref["margin"] < FLAG  # NaN (greedy, unusable) is never flagged
    bad = np.nonzero(mism & ~flagged)[0]
    assert bad.size == 0, (f"{label}: {bad.size} unflagged mismatches, first rows {bad[:5].tolist()}: "
                           f"gpu {got[bad[:5]].tolist()} oracle {ref['tokens'][bad[:5]].tolist()}")
    assert mism.sum() <= int(1e-4 * rows), f"{label}: {mism.sum()} flagged mismatches of {rows} rows"
    return got, ref


def test_sampler_large_draft_rows(sv):
    """The 1280 draft rows of the large verify workload (bf16 Student-t, V=128256), T = 1."""
    d = inputgen.make("large")
    rows = d["draft"].reshape(-1, d["draft"].shape[-1])
    u = inputgen.uniform24(31, inputgen.S_USAMP, rows.shape[0])
    got, ref = check(sv, rows, 1.0, u, "large-draft")
    assert (got >= 0).all()


def test_sampler_mid_rows(sv):
    d = inputgen.make("mid")  # fp32, V=32000, 20 spikes per row
    rows = d["target"].reshape(-1, d["target"].shape[-1])
    check(sv, rows, 0.8, inputgen.uniform24(32, inputgen.S_USAMP, rows.shape[0]), "mid")


def test_sampler_mixed_temperatures(sv):
    """bf16 N(0, 3) rows at V=151936: a quarter greedy, the rest T ~ U(0.5, 1.2)."""
    n = 512
    rows = inputgen.logit_rows(33, 151936, np.arange(n, dtype=np.int64), scale=3.0, dtype="bf16")
    T = (0.5 + 0.7 * inputgen.uniform53(33, inputgen.S_USAMP + 1, n)).astype(np.float32)
    T[::4] = 0.0
    got, ref = check(sv, rows, T, inputgen.uniform24(33, inputgen.S_USAMP, n), "mixed-T")
    assert (got[::4] == ref["tokens"][::4]).all()


@pytest.mark.parametrize("dtype,V", [("f32", 1), ("bf16", 1), ("f32", 7), ("bf16", 7), ("f32", 2049),
                                     ("bf16", 4097), ("f32", 20001), ("bf16", 131075), ("f32", 300007),
                                     ("bf16", 600001)])
def test_sampler_shapes(sv, dtype, V):
    """Ragged vocabulary tails; odd bf16 V leaves rows off the 16-byte grid; the two largest rows
    hold more than 256 sampling tiles (the pick reads the tile records from memory)."""
    n = 37
    rows = inputgen.logit_rows(34 + V, V, np.arange(n, dtype=np.int64), scale=2.0, dtype=dtype)
    check(sv, rows, 1.0, inputgen.uniform24(34, inputgen.S_USAMP, n), f"{dtype}-V{V}")


def test_sampler_temperature_extremes(sv):
    n = 64
    rows = inputgen.logit_rows(35, 5000, np.arange(n, dtype=np.int64), scale=3.0, dtype="f32")
    T = np.array([1e-30, 1e-3, 0.05, 1.0, 50.0, 1e6, 1e30, 1.17549435e-38] * 8, np.float32)
    check(sv, rows, T, inputgen.uniform24(35, inputgen.S_USAMP, n), "T-extremes")


def test_sampler_unusable_rows(sv):
    rows = inputgen.logit_rows(36, 300, np.arange(8, dtype=np.int64), scale=1.0, dtype="f32")
    rows[5, 17] = np.nan
    rows[6, :] = -np.inf
    rows[7, 3] = np.inf
    T = np.array([np.nan, -1.0, 1e-40, 1.0, 1.0, 1.0, 1.0, 1.0], np.float32)
    u = np.array([0.5, 0.5, 0.5, 1.0, np.nan, 0.5, 0.5, 0.5], np.float32)
    got, _ = check(sv, rows, T, u, "unusable")
    assert got.tolist() == [-1] * 8


def test_sampler_is_deterministic(sv):
    d = inputgen.make("tiny")
    rows = d["target"].reshape(-1, d["target"].shape[-1])
    u = inputgen.uniform24(37, inputgen.S_USAMP, rows.shape[0])
    a, _ = check(sv, rows, 1.0, u, "det-a")
    b, _ = check(sv, rows, 1.0, u, "det-b")
    assert np.array_equal(a, b)
