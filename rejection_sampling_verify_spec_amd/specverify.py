"""Thin ctypes binding of libspecverify (see include/specverify.h).

The functions named like the C entry points marshal torch device tensors into
pointers and pass torch's current HIP stream; every step of the verify path
runs in the HIP kernels of the library. There is no fallback: if the built
library is missing, importing this module raises.

The convenience wrappers (``verify_chain``, ``verify_ragged``, ``verify_tree``,
``row_softmax_stats``) only allocate outputs and a workspace with torch.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; SPECVERIFY_LIB names another build of the same library
LIB_PATH = os.environ.get("SPECVERIFY_LIB") or os.path.join(_HERE, "libspecverify.so")

SV_OK, SV_EINVAL, SV_EDTYPE, SV_ENOWS, SV_EALIGN, SV_EHIP, SV_ESCRATCH = 0, -1, -2, -3, -4, -5, -6
SV_NOALLOC_SCRATCH_BYTES = 32 << 20
SV_F32, SV_BF16 = 0, 1

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build() "
                      "(or python rejection_sampling_verify_spec_amd/build.py)")

_lib = ctypes.CDLL(LIB_PATH)
_P, _I32, _SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t

_lib.spec_verify_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
_lib.spec_verify_workspace_bytes.restype = _SZ
_lib.spec_verify_ragged_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32, _I32]
_lib.spec_verify_ragged_workspace_bytes.restype = _SZ
_lib.spec_verify_tree_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
_lib.spec_verify_tree_workspace_bytes.restype = _SZ
_lib.spec_row_softmax_stats_workspace_bytes.argtypes = [_I32, _I32, _I32]
_lib.spec_row_softmax_stats_workspace_bytes.restype = _SZ
_lib.spec_verify.argtypes = [_P, _P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]
_lib.spec_verify.restype = ctypes.c_int
_lib.spec_verify_noalloc.argtypes = [_P, _P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P]
_lib.spec_verify_noalloc.restype = ctypes.c_int
_lib.spec_verify_ragged.argtypes = [_P, _P, _I32, _P, _I32, _P, _P, _P, _P, _I32, _I32, _I32, _P, _P, _P, _P, _SZ,
                                    _P]
_lib.spec_verify_ragged.restype = ctypes.c_int
_lib.spec_verify_tree.argtypes = [_P, _P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]
_lib.spec_verify_tree.restype = ctypes.c_int
_lib.spec_verify_tree_lossless_workspace_bytes.argtypes = [_I32, _I32, _I32, _I32]
_lib.spec_verify_tree_lossless_workspace_bytes.restype = _SZ
_lib.spec_verify_tree_lossless.argtypes = [_P, _P, _I32, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _P, _P, _P, _P,
                                           _SZ, _P]
_lib.spec_verify_tree_lossless.restype = ctypes.c_int
_lib.spec_row_softmax_stats.argtypes = [_P, _I32, _I32, _I32, _P, _P, _P, _P, _P, _SZ, _P]
_lib.spec_row_softmax_stats.restype = ctypes.c_int
_lib.spec_sample_rows_workspace_bytes.argtypes = [_I32, _I32, _I32]
_lib.spec_sample_rows_workspace_bytes.restype = _SZ
_lib.spec_sample_rows.argtypes = [_P, _I32, _I32, _I32, _P, _P, _P, _P, _SZ, _P]
_lib.spec_sample_rows.restype = ctypes.c_int
_I64 = ctypes.c_int64
_lib.spec_kv_commit.argtypes = [_P, _P, _P, _P, _P, _P, _P, _I32, _I32, _I32, _I64, _I32, _I32, _P]
_lib.spec_kv_commit.restype = ctypes.c_int
_lib.spec_kv_valid_slots.argtypes = [_P, _I32, _I32, _I32, _P, _P, _P, _P]
_lib.spec_kv_valid_slots.restype = ctypes.c_int
_lib.spec_draft_window_max_blocks.argtypes = [_I32, _I32]
_lib.spec_draft_window_max_blocks.restype = _I32
_lib.spec_draft_window.argtypes = [_P, _I32, _I32, _I32, _I32, _P, _I32, _P, _P, _I32, _P]
_lib.spec_draft_window.restype = ctypes.c_int
_lib.spec_draft_window_host.argtypes = [_P, _I32, _I32, _I32, _I32, _P]
_lib.spec_draft_window_host.restype = ctypes.c_int
_lib.spec_read_probe_words.argtypes = [_SZ]
_lib.spec_read_probe_words.restype = _SZ
_lib.spec_read_probe.argtypes = [_P, _SZ, _P, _P]
_lib.spec_read_probe.restype = ctypes.c_int
_lib.spec_verify_strerror.argtypes = [ctypes.c_int]
_lib.spec_verify_strerror.restype = ctypes.c_char_p
_lib.spec_verify_version.restype = ctypes.c_int
_lib.spec_verify_timing_enable.argtypes = [ctypes.c_int]
_lib.spec_verify_timing_enable.restype = ctypes.c_int
_lib.spec_verify_timing_reset.argtypes = []
_lib.spec_verify_timing_reset.restype = ctypes.c_int
_lib.spec_verify_timing_read.argtypes = [_P, _I32, _P]
_lib.spec_verify_timing_read.restype = ctypes.c_int


class SpecVerifyError(RuntimeError):
    pass


def _check(rc: int) -> None:
    if rc != SV_OK:
        raise SpecVerifyError(f"libspecverify: {spec_verify_strerror(rc)} ({rc})")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(device=None):
    return torch.cuda.current_stream(device).cuda_stream


def logits_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SV_F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return SV_BF16
    raise TypeError(f"logits must be float32 or bfloat16 (got {t.dtype})")


# ---------------------------------------------------------------------------
# Entry points with the C names (pointers may be tensors or raw ints)


def spec_verify_strerror(status: int) -> str:
    return _lib.spec_verify_strerror(int(status)).decode()


def spec_verify_version() -> int:
    return _lib.spec_verify_version()


def spec_verify_workspace_bytes(B, gamma, V, dtype) -> int:
    return _lib.spec_verify_workspace_bytes(B, gamma, V, dtype)


def spec_verify_ragged_workspace_bytes(B, total_draft, gamma_max, V, dtype) -> int:
    return _lib.spec_verify_ragged_workspace_bytes(B, total_draft, gamma_max, V, dtype)


def spec_verify_tree_workspace_bytes(B, N, V, dtype) -> int:
    return _lib.spec_verify_tree_workspace_bytes(B, N, V, dtype)


def spec_verify_tree_lossless_workspace_bytes(B, N, V, dtype) -> int:
    return _lib.spec_verify_tree_lossless_workspace_bytes(B, N, V, dtype)


def spec_row_softmax_stats_workspace_bytes(rows, V, dtype) -> int:
    return _lib.spec_row_softmax_stats_workspace_bytes(rows, V, dtype)


def spec_verify(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, temperature, B, gamma, V,
                out_tokens, num_accepted, diag_probs, workspace, workspace_bytes, stream) -> int:
    return _lib.spec_verify(_ptr(target_logits), _ptr(draft_logits), dtype, _ptr(draft_tokens), _ptr(u_accept),
                            _ptr(u_sample), _ptr(temperature), B, gamma, V, _ptr(out_tokens), _ptr(num_accepted),
                            _ptr(diag_probs), _ptr(workspace), workspace_bytes, stream)


def spec_verify_noalloc(target_logits, draft_logits, dtype, draft_tokens, u_accept, u_sample, temperature, B, gamma,
                        V, out_tokens, num_accepted, diag_probs, stream) -> int:
    return _lib.spec_verify_noalloc(_ptr(target_logits), _ptr(draft_logits), dtype, _ptr(draft_tokens),
                                    _ptr(u_accept), _ptr(u_sample), _ptr(temperature), B, gamma, V, _ptr(out_tokens),
                                    _ptr(num_accepted), _ptr(diag_probs), stream)


def spec_verify_ragged(target_logits, draft_logits, dtype, cu_gamma, total_draft, draft_tokens, u_accept, u_sample,
                       temperature, B, gamma_max, V, out_tokens, num_accepted, diag_probs, workspace,
                       workspace_bytes, stream) -> int:
    return _lib.spec_verify_ragged(_ptr(target_logits), _ptr(draft_logits), dtype, _ptr(cu_gamma), total_draft,
                                   _ptr(draft_tokens), _ptr(u_accept), _ptr(u_sample), _ptr(temperature), B,
                                   gamma_max, V, _ptr(out_tokens), _ptr(num_accepted), _ptr(diag_probs),
                                   _ptr(workspace), workspace_bytes, stream)


def spec_verify_tree(target_logits, draft_logits, dtype, node_tokens, parents, u_accept, u_sample, temperature, B, N,
                     V, max_depth, out_tokens, out_nodes, num_accepted, workspace, workspace_bytes, stream) -> int:
    return _lib.spec_verify_tree(_ptr(target_logits), _ptr(draft_logits), dtype, _ptr(node_tokens), _ptr(parents),
                                 _ptr(u_accept), _ptr(u_sample), _ptr(temperature), B, N, V, max_depth,
                                 _ptr(out_tokens), _ptr(out_nodes), _ptr(num_accepted), _ptr(workspace),
                                 workspace_bytes, stream)


def spec_verify_tree_lossless(target_logits, draft_logits, dtype, node_tokens, parents, u_accept, u_sample,
                              temperature, B, N, V, max_depth, out_tokens, out_nodes, num_accepted, workspace,
                              workspace_bytes, stream) -> int:
    return _lib.spec_verify_tree_lossless(_ptr(target_logits), _ptr(draft_logits), dtype, _ptr(node_tokens),
                                          _ptr(parents), _ptr(u_accept), _ptr(u_sample), _ptr(temperature), B, N, V,
                                          max_depth, _ptr(out_tokens), _ptr(out_nodes), _ptr(num_accepted),
                                          _ptr(workspace), workspace_bytes, stream)


def spec_row_softmax_stats(logits, dtype, rows, V, temperature, out_max, out_logz, out_argmax, workspace,
                           workspace_bytes, stream) -> int:
    return _lib.spec_row_softmax_stats(_ptr(logits), dtype, rows, V, _ptr(temperature), _ptr(out_max),
                                       _ptr(out_logz), _ptr(out_argmax), _ptr(workspace), workspace_bytes, stream)


def spec_sample_rows_workspace_bytes(rows, V, dtype) -> int:
    return _lib.spec_sample_rows_workspace_bytes(rows, V, dtype)


def spec_sample_rows(logits, dtype, rows, V, temperature, u, out_tokens, workspace, workspace_bytes, stream) -> int:
    return _lib.spec_sample_rows(_ptr(logits), dtype, rows, V, _ptr(temperature), _ptr(u), _ptr(out_tokens),
                                 _ptr(workspace), workspace_bytes, stream)


def spec_read_probe_words(nbytes) -> int:
    return _lib.spec_read_probe_words(nbytes)


def spec_read_probe(src, nbytes, out, stream) -> int:
    return _lib.spec_read_probe(_ptr(src), nbytes, _ptr(out), stream)


def read_probe(t, out=None):
    """Read every byte of device tensor t with the streaming kernel's load pattern (a measurement aid)."""
    nbytes = t.numel() * t.element_size() // 16 * 16
    if out is None:
        out = torch.empty(max(spec_read_probe_words(nbytes), 1), dtype=torch.int32, device=t.device)
    _check(spec_read_probe(t, nbytes, out, _stream(t.device)))
    return out


def spec_kv_commit(k_cache, v_cache, k_new, v_new, lengths, num_accepted, new_lengths, B, gamma, rows, row_bytes,
                   sink, window, stream) -> int:
    return _lib.spec_kv_commit(_ptr(k_cache), _ptr(v_cache), _ptr(k_new), _ptr(v_new), _ptr(lengths),
                               _ptr(num_accepted), _ptr(new_lengths), B, gamma, rows, row_bytes, sink, window, stream)


def spec_kv_valid_slots(lengths, B, sink, window, slots, positions, counts, stream) -> int:
    return _lib.spec_kv_valid_slots(_ptr(lengths), B, sink, window, _ptr(slots), _ptr(positions), _ptr(counts),
                                    stream)


def spec_draft_window_max_blocks(window, block_size) -> int:
    return _lib.spec_draft_window_max_blocks(window, block_size)


def spec_draft_window(seq_lens, B, window, block_size, future_offset, block_table, full_cols, windowed_lens,
                      window_table, window_cols, stream) -> int:
    return _lib.spec_draft_window(_ptr(seq_lens), B, window, block_size, future_offset, _ptr(block_table), full_cols,
                                  _ptr(windowed_lens), _ptr(window_table), window_cols, stream)


def spec_draft_window_host(seq_lens, n, window, block_size, future_offset, windowed_lens) -> int:
    return _lib.spec_draft_window_host(_ptr(seq_lens), n, window, block_size, future_offset, _ptr(windowed_lens))


def spec_verify_timing_enable(enable: bool) -> int:
    """Start/resume (True) or pause (False) event timing of the row-statistics kernel."""
    return _lib.spec_verify_timing_enable(1 if enable else 0)


def spec_verify_timing_reset() -> int:
    """Forget the recorded durations."""
    return _lib.spec_verify_timing_reset()


def spec_verify_timing_read(max_n: int = 4096):
    """Recorded per-call durations (ms) of the row-statistics kernel."""
    buf = (ctypes.c_float * max_n)()
    cnt = ctypes.c_int32(0)
    _check(_lib.spec_verify_timing_read(ctypes.cast(buf, _P), max_n, ctypes.addressof(cnt)))
    return [buf[i] for i in range(min(cnt.value, max_n))]


# ---------------------------------------------------------------------------
# Allocating wrappers


class Workspace:
    """A reusable, 256-byte aligned device workspace that grows on demand."""

    def __init__(self, device="cuda"):
        self.device = torch.device(device)
        self.buf = None

    def get(self, nbytes: int) -> torch.Tensor:
        if self.buf is None or self.buf.numel() < nbytes:
            self.buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        return self.buf


_default_ws = {}


def _ws(device, nbytes):
    key = str(device)
    if key not in _default_ws:
        _default_ws[key] = Workspace(device)
    return _default_ws[key].get(nbytes)


def _need(t, dtype, name):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def verify_chain(target, draft, draft_tokens, u_accept, u_sample, temperature, *, diag=False, workspace=None):
    """Dense verify. target [B, g+1, V], draft [B, g, V]; returns (out_tokens, num_accepted[, diag])."""
    B, g1, V = target.shape
    g = g1 - 1
    dt = logits_dtype(target)
    for t, n in ((target, "target"), (draft, "draft")):
        _need(t, None, n)
    for t, n in ((draft_tokens, "draft_tokens"),):
        _need(t, torch.int32, n)
    for t, n in ((u_accept, "u_accept"), (u_sample, "u_sample"), (temperature, "temperature")):
        _need(t, torch.float32, n)
    dev = target.device
    out = torch.empty((B, g + 1), dtype=torch.int32, device=dev)
    na = torch.empty(B, dtype=torch.int32, device=dev)
    dg = torch.empty((B, g, 2), dtype=torch.float32, device=dev) if diag else None
    nbytes = spec_verify_workspace_bytes(B, g, V, dt)
    ws = workspace if workspace is not None else _ws(dev, nbytes)
    _check(spec_verify(target, draft, dt, draft_tokens, u_accept, u_sample, temperature, B, g, V, out, na, dg, ws,
                       ws.numel(), _stream(dev)))
    return (out, na, dg) if diag else (out, na)


def verify_ragged(target, draft, cu_gamma, total_draft, draft_tokens, u_accept, u_sample, temperature, gamma_max, *,
                  diag=False, workspace=None):
    """Ragged verify (packed rows, cu_gamma [B+1]); returns (out_tokens [B, gmax+1], num_accepted[, diag])."""
    V = target.shape[-1]
    B = temperature.shape[0]
    dt = logits_dtype(target)
    _need(target, None, "target")
    _need(cu_gamma, torch.int32, "cu_gamma")
    dev = target.device
    out = torch.empty((B, gamma_max + 1), dtype=torch.int32, device=dev)
    na = torch.empty(B, dtype=torch.int32, device=dev)
    dg = torch.empty((max(total_draft, 1), 2), dtype=torch.float32, device=dev) if diag else None
    nbytes = spec_verify_ragged_workspace_bytes(B, total_draft, gamma_max, V, dt)
    ws = workspace if workspace is not None else _ws(dev, nbytes)
    _check(spec_verify_ragged(target, draft, dt, cu_gamma, total_draft, draft_tokens, u_accept, u_sample, temperature,
                              B, gamma_max, V, out, na, dg, ws, ws.numel(), _stream(dev)))
    return (out, na, dg) if diag else (out, na)


def verify_tree(target, draft, node_tokens, parents, u_accept, u_sample, temperature, max_depth, *, workspace=None):
    """Tree verify. target [B, N, V], draft [B, N-1, V]; returns (out_tokens, out_nodes, num_accepted)."""
    B, N, V = target.shape
    dt = logits_dtype(target)
    _need(target, None, "target")
    dev = target.device
    out = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    nodes = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    na = torch.empty(B, dtype=torch.int32, device=dev)
    nbytes = spec_verify_tree_workspace_bytes(B, N, V, dt)
    ws = workspace if workspace is not None else _ws(dev, nbytes)
    _check(spec_verify_tree(target, draft, dt, node_tokens, parents, u_accept, u_sample, temperature, B, N, V,
                            max_depth, out, nodes, na, ws, ws.numel(), _stream(dev)))
    return out, nodes, na


def verify_tree_lossless(target, draft, node_tokens, parents, u_accept, u_sample, temperature, max_depth, *,
                         workspace=None):
    """Lossless multi-candidate tree verify (siblings tried in order against the running residual).
    target [B, N, V], draft [B, N-1, V]; returns (out_tokens, out_nodes, num_accepted)."""
    B, N, V = target.shape
    dt = logits_dtype(target)
    _need(target, None, "target")
    dev = target.device
    out = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    nodes = torch.empty((B, max_depth + 1), dtype=torch.int32, device=dev)
    na = torch.empty(B, dtype=torch.int32, device=dev)
    nbytes = spec_verify_tree_lossless_workspace_bytes(B, N, V, dt)
    ws = workspace if workspace is not None else _ws(dev, nbytes)
    _check(spec_verify_tree_lossless(target, draft, dt, node_tokens, parents, u_accept, u_sample, temperature, B, N,
                                     V, max_depth, out, nodes, na, ws, ws.numel(), _stream(dev)))
    return out, nodes, na


def row_softmax_stats(logits, temperature, *, workspace=None):
    """Per-row (max, log-partition, greedy argmax) of logits [rows, V]."""
    V = logits.shape[-1]
    rows = logits.numel() // V
    dt = logits_dtype(logits)
    dev = logits.device
    mx = torch.empty(rows, dtype=torch.float32, device=dev)
    lz = torch.empty(rows, dtype=torch.float32, device=dev)
    am = torch.empty(rows, dtype=torch.int32, device=dev)
    nbytes = spec_row_softmax_stats_workspace_bytes(rows, V, dt)
    ws = workspace if workspace is not None else _ws(dev, nbytes)
    _check(spec_row_softmax_stats(logits, dt, rows, V, temperature, mx, lz, am, ws, ws.numel(), _stream(dev)))
    return mx, lz, am


def sample_rows(logits, temperature, u, *, workspace=None):
    """One token per row of logits [rows, V] from softmax(l/T) with the caller's uniforms (T == 0: argmax)."""
    V = logits.shape[-1]
    rows = logits.numel() // V if V else 0
    dt = logits_dtype(logits)
    _need(logits, None, "logits")
    _need(temperature, torch.float32, "temperature")
    _need(u, torch.float32, "u")
    dev = logits.device
    out = torch.empty(rows, dtype=torch.int32, device=dev)
    nbytes = spec_sample_rows_workspace_bytes(rows, V, dt)
    ws = workspace if workspace is not None else _ws(dev, nbytes)
    _check(spec_sample_rows(logits, dt, rows, V, temperature, u, out, ws, ws.numel(), _stream(dev)))
    return out


def kv_commit(k_cache, v_cache, k_new, v_new, lengths, num_accepted, sink, window):
    """Commit the kept positions of one verify step into sink + ring caches.

    k_cache, v_cache [B, R, S+W, ...] (updated in place), k_new, v_new [B, gamma+1, R, ...] with the same
    trailing shape and dtype, lengths and num_accepted int32 [B]. Returns the new lengths."""
    B, R, cap = k_cache.shape[:3]
    if cap != sink + window:
        raise ValueError(f"cache has {cap} slots, sink + window = {sink + window}")
    gamma = k_new.shape[1] - 1
    for name, t in (("k_cache", k_cache), ("v_cache", v_cache), ("k_new", k_new), ("v_new", v_new)):
        _need(t, k_cache.dtype, name)
    if tuple(v_cache.shape) != tuple(k_cache.shape) or tuple(v_new.shape) != tuple(k_new.shape) or \
            tuple(k_new.shape[:1] + k_new.shape[2:3]) != (B, R) or k_new.shape[3:] != k_cache.shape[3:]:
        raise ValueError("cache and staging shapes do not match")
    _need(lengths, torch.int32, "lengths")
    _need(num_accepted, torch.int32, "num_accepted")
    row_bytes = math.prod(k_cache.shape[3:]) * k_cache.element_size()
    out = torch.empty_like(lengths)
    _check(spec_kv_commit(k_cache, v_cache, k_new, v_new, lengths, num_accepted, out, B, gamma, R, row_bytes, sink,
                          window, _stream(k_cache.device)))
    return out


def kv_valid_slots(lengths, sink, window, *, positions=True):
    """(slots [B, S+W], positions [B, S+W] or None, counts [B]) of sink + ring caches of these lengths."""
    _need(lengths, torch.int32, "lengths")
    B = lengths.shape[0]
    dev = lengths.device
    slots = torch.empty((B, sink + window), dtype=torch.int32, device=dev)
    pos = torch.empty_like(slots) if positions else None
    counts = torch.empty(B, dtype=torch.int32, device=dev)
    _check(spec_kv_valid_slots(lengths, B, sink, window, slots, pos, counts, _stream(dev)))
    return slots, pos, counts


def draft_window(seq_lens, block_table, window, block_size, future_offset, *, window_cols=None):
    """(windowed_lens [B], window_table [B, window_cols]) of a draft KV window over a full block table [B, cols]."""
    _need(seq_lens, torch.int32, "seq_lens")
    _need(block_table, torch.int32, "block_table")
    B = seq_lens.shape[0]
    dev = seq_lens.device
    cols = window_cols if window_cols is not None else spec_draft_window_max_blocks(window, block_size)
    lens = torch.empty(B, dtype=torch.int32, device=dev)
    table = torch.empty((B, max(cols, 0)), dtype=torch.int32, device=dev)
    _check(spec_draft_window(seq_lens, B, window, block_size, future_offset, block_table, block_table.shape[1], lens,
                             table, cols, _stream(dev)))
    return lens, table
