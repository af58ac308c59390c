"""Helpers for GPU parity tests: moving generator outputs to the device, and the
acceptance bar for sampled tokens.

Bar: out_tokens and num_accepted equal the oracle's bit for bit; a request may
differ only when the oracle flags it as a near-tie (a uniform within 1e-5 of
its acceptance ratio, or u*S within 1e-5*S of a CDF boundary), and such
requests must stay below 1e-4 of all requests (zero for batches under 10^4).
Per-position probabilities agree within 1e-5 (fp32 logits) or 2e-3 (bf16
logits) in relative terms, checked as |log p_gpu - log p_oracle|.
"""
import numpy as np

FLAG = 1e-5


def to_dev(a, dev="cuda"):
    import torch
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def device_inputs(d, dev="cuda"):
    return {k: to_dev(v, dev) for k, v in d.items() if isinstance(v, np.ndarray)}


def assert_tokens_match(out, na, ref, label=""):
    out = np.asarray(out)
    na = np.asarray(na)
    B = na.shape[0]
    mism = (na != ref["num_accepted"]) | (out != ref["out_tokens"]).any(axis=1)
    flagged = (ref["acc_margin"] < FLAG) | (ref["cdf_margin"] < FLAG)
    bad = np.nonzero(mism & ~flagged)[0]
    assert bad.size == 0, (f"{label}: {bad.size} unflagged mismatches, first {bad[:5].tolist()}; "
                           f"gpu {out[bad[:3]].tolist()} / {na[bad[:3]].tolist()} vs oracle "
                           f"{ref['out_tokens'][bad[:3]].tolist()} / {ref['num_accepted'][bad[:3]].tolist()}")
    assert mism.sum() <= int(1e-4 * B), f"{label}: {mism.sum()} flagged mismatches of {B} requests"
    return int(mism.sum())


def assert_probs_match(diag, ref, rows_valid, tol, label=""):
    """diag [rows, 2] (p_t, p_d) from the GPU against the oracle's p_t/p_d at valid rows."""
    diag = np.asarray(diag, np.float64).reshape(-1, 2)
    pt, pd = ref["p_t"], ref["p_d"]
    for k, (g, o) in enumerate(((diag[:, 0], pt), (diag[:, 1], pd))):
        g, o = g[rows_valid], o[rows_valid]
        tiny = (o < 1.2e-38) & (g < 1.2e-38)
        with np.errstate(divide="ignore"):
            err = np.abs(np.log(g) - np.log(o))
        err[tiny] = 0.0
        assert np.all(err <= tol), (f"{label}: {'p_t' if k == 0 else 'p_d'} rel err {err.max():.3g} > {tol} "
                                    f"at {np.argmax(err)}")
