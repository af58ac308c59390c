"""CPU fp64 oracle for batched speculative-decoding verification.

TEST INFRASTRUCTURE: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` import this package. The HIP library never
loads it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, double precision, ascending
loops); this module only builds it with gcc and marshals numpy arrays.
Function-level citations are in ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

F32, BF16 = 0, 1
MUT_NONE, MUT_LOGIT_RESIDUAL, MUT_RESAMPLE_TARGET, MUT_ALWAYS_ACCEPT, MUT_NO_BONUS = range(5)
MUT_TREE_NO_UPDATE, MUT_TREE_NO_RENORM = 5, 6

_lib = None


def _compiler():
    """gcc, or with SPECVERIFY_SANITIZE=1 ROCm's clang with AddressSanitizer and UndefinedBehaviorSanitizer."""
    if os.environ.get("SPECVERIFY_SANITIZE") == "1":
        return ["/opt/rocm/llvm/bin/clang", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
                "-fno-omit-frame-pointer", "-shared-libsan", "-g"]
    return ["gcc"]


def build(force: bool = True) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp"
        cmd = _compiler() + ["-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off", "-fno-fast-math",
                             "-pthread", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        lib.oracle_verify_chain.argtypes = [P, P, I, P, P, P, P, P, I, I, I, I, P, P, P, P, P, P, P, I, I]
        lib.oracle_verify_chain.restype = I
        lib.oracle_verify_tree.argtypes = [P, P, I, P, P, P, P, P, I, I, I, I, P, P, P, P, P, P, I]
        lib.oracle_verify_tree.restype = I
        lib.oracle_verify_tree_lossless.argtypes = [P, P, I, P, P, P, P, P, I, I, I, I, P, P, P, P, P, P, I, I]
        lib.oracle_verify_tree_lossless.restype = I
        lib.oracle_row_stats.argtypes = [P, I, I, I, P, P, P, P, P, I]
        lib.oracle_row_stats.restype = I
        lib.oracle_sample_rows.argtypes = [P, I, I, I, P, P, P, P, I]
        lib.oracle_sample_rows.restype = I
        _lib = lib
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    if n:
        return int(n)
    return max(1, min(16, os.cpu_count() or 1))


def _logits(a):
    """Accept float32 arrays or bf16 stored as uint16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError("logits must be float32 or uint16 (bf16 bits)")


def verify_chain(target, draft, draft_tokens, u_accept, u_sample, temperature, *, gamma=None,
                 cu_gamma=None, mutant=MUT_NONE, nthreads=None):
    """Dense (cu_gamma None) or ragged chain verification.

    Dense: target [B, g+1, V], draft [B, g, V], draft_tokens/u_accept [B, g],
    u_sample [B, g+1]. Ragged: target [sum(g_b+1), V], draft [sum g_b, V],
    packed 1-D token/uniform arrays, cu_gamma [B+1], ``gamma`` = g_max.
    Returns dict(out_tokens [B, g+1], num_accepted [B], p_t, p_d (per draft row),
    acc_margin [B], cdf_margin [B], fallback [B]: True where the residual summed to 0 and the
    draw fell back to P_t of the same row).
    """
    target, dt = _logits(target)
    draft, dt2 = _logits(draft)
    assert dt == dt2
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    B = temperature.shape[0]
    V = target.shape[-1]
    tokens = np.ascontiguousarray(draft_tokens, dtype=np.int32).reshape(-1)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32).reshape(-1)
    us = np.ascontiguousarray(u_sample, dtype=np.float32).reshape(-1)
    if cu_gamma is None:
        g = int(draft_tokens.shape[1]) if gamma is None else int(gamma)
        cu = None
        total = B * g
    else:
        cu = np.ascontiguousarray(cu_gamma, dtype=np.int32)
        g = int(gamma)
        total = int(tokens.shape[0])
    out = np.empty((B, g + 1), np.int32)
    na = np.empty(B, np.int32)
    pt = np.empty(total, np.float64)
    pd = np.empty(total, np.float64)
    am = np.empty(B, np.float64)
    cm = np.empty(B, np.float64)
    fb = np.empty(B, np.int32)
    rc = _load().oracle_verify_chain(_ptr(target), _ptr(draft), dt, _ptr(tokens), _ptr(ua), _ptr(us),
                                     _ptr(temperature), _ptr(cu), total, B, g, V, _ptr(out), _ptr(na),
                                     _ptr(pt), _ptr(pd), _ptr(am), _ptr(cm), _ptr(fb), int(mutant),
                                     _threads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_verify_chain failed")
    return dict(out_tokens=out, num_accepted=na, p_t=pt, p_d=pd, acc_margin=am, cdf_margin=cm,
                fallback=fb.astype(bool))


def verify_tree(target, draft, node_tokens, parents, u_accept, u_sample, temperature, max_depth,
                nthreads=None):
    """Token-tree verification. target [B, N, V]; draft [B, N-1, V] (row v-1 is node v);
    node_tokens, parents, u_accept, u_sample [B, N]. Returns dict(out_tokens,
    out_nodes [B, max_depth+1], num_accepted [B], acc_margin, cdf_margin, fallback: True where the
    residual at the end node summed to 0 and the draw fell back to its target row)."""
    target, dt = _logits(target)
    draft, dt2 = _logits(draft)
    assert dt == dt2
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    B, N, V = target.shape
    tok = np.ascontiguousarray(node_tokens, dtype=np.int32)
    par = np.ascontiguousarray(parents, dtype=np.int32)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32)
    us = np.ascontiguousarray(u_sample, dtype=np.float32)
    out = np.empty((B, max_depth + 1), np.int32)
    onodes = np.empty((B, max_depth + 1), np.int32)
    na = np.empty(B, np.int32)
    am = np.empty(B, np.float64)
    cm = np.empty(B, np.float64)
    fb = np.empty(B, np.int32)
    rc = _load().oracle_verify_tree(_ptr(target), _ptr(draft), dt, _ptr(tok), _ptr(par), _ptr(ua), _ptr(us),
                                    _ptr(temperature), B, N, V, int(max_depth), _ptr(out), _ptr(onodes),
                                    _ptr(na), _ptr(am), _ptr(cm), _ptr(fb), _threads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_verify_tree failed")
    return dict(out_tokens=out, out_nodes=onodes, num_accepted=na, acc_margin=am, cdf_margin=cm,
                fallback=fb.astype(bool))


def verify_tree_lossless(target, draft, node_tokens, parents, u_accept, u_sample, temperature, max_depth,
                         nthreads=None, mutant=MUT_NONE):
    """Lossless multi-candidate token-tree verification (siblings tried in index order, each
    against the residual left by the rejected ones). Same arguments and outputs as verify_tree;
    fallback is True where a rejected sibling's residual summed to 0 and r was kept."""
    target, dt = _logits(target)
    draft, dt2 = _logits(draft)
    assert dt == dt2
    temperature = np.ascontiguousarray(temperature, dtype=np.float32)
    B, N, V = target.shape
    tok = np.ascontiguousarray(node_tokens, dtype=np.int32)
    par = np.ascontiguousarray(parents, dtype=np.int32)
    ua = np.ascontiguousarray(u_accept, dtype=np.float32)
    us = np.ascontiguousarray(u_sample, dtype=np.float32)
    out = np.empty((B, max_depth + 1), np.int32)
    onodes = np.empty((B, max_depth + 1), np.int32)
    na = np.empty(B, np.int32)
    am = np.empty(B, np.float64)
    cm = np.empty(B, np.float64)
    fb = np.empty(B, np.int32)
    rc = _load().oracle_verify_tree_lossless(_ptr(target), _ptr(draft), dt, _ptr(tok), _ptr(par), _ptr(ua),
                                             _ptr(us), _ptr(temperature), B, N, V, int(max_depth), _ptr(out),
                                             _ptr(onodes), _ptr(na), _ptr(am), _ptr(cm), _ptr(fb), int(mutant),
                                             _threads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_verify_tree_lossless failed")
    return dict(out_tokens=out, out_nodes=onodes, num_accepted=na, acc_margin=am, cdf_margin=cm,
                fallback=fb.astype(bool))


def row_stats(logits, temperature, nthreads=None):
    """Per-row max, log-partition log sum exp((l-m)/T) (T>0) and lowest argmax (T==0)."""
    logits, dt = _logits(logits)
    V = logits.shape[-1]
    rows = logits.size // V
    temperature = np.ascontiguousarray(np.broadcast_to(np.asarray(temperature, np.float32), (rows,)))
    m = np.empty(rows, np.float64)
    lz = np.empty(rows, np.float64)
    am = np.empty(rows, np.int32)
    valid = np.empty(rows, np.int32)
    rc = _load().oracle_row_stats(_ptr(logits), dt, rows, V, _ptr(temperature), _ptr(m), _ptr(lz), _ptr(am),
                                  _ptr(valid), _threads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_row_stats failed")
    return dict(max=m, logz=lz, argmax=am, valid=valid.astype(bool))


def sample_rows(logits, temperature, u, nthreads=None):
    """One token per row from softmax(l/T) by the inverse-CDF rule (T == 0: lowest argmax).

    Returns tokens (int32, -1 for unusable rows) and the CDF margin (distance of u*S to the
    nearer edge of the chosen token's interval, over S; NaN for greedy and unusable rows).
    """
    logits, dt = _logits(logits)
    V = logits.shape[-1]
    rows = logits.size // V
    temperature = np.ascontiguousarray(np.broadcast_to(np.asarray(temperature, np.float32), (rows,)))
    u = np.ascontiguousarray(np.broadcast_to(np.asarray(u, np.float32), (rows,)))
    out = np.empty(rows, np.int32)
    margin = np.empty(rows, np.float64)
    rc = _load().oracle_sample_rows(_ptr(logits), dt, rows, V, _ptr(temperature), _ptr(u), _ptr(out),
                                    _ptr(margin), _threads(nthreads))
    if rc != 0:
        raise RuntimeError("oracle_sample_rows failed")
    return dict(tokens=out, margin=margin)


# KV-cache steps around verification (plain Python/numpy, no C)
from .cache import (  # noqa: E402,F401
    draft_window, kv_commit, kv_valid_slots, max_window_blocks, slot, valid_slots, window_one,
)
