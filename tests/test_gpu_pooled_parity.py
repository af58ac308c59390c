"""Pooled GPU parity over many seeds (seeds 1000 + k): the near-tie part of the parity bar is a rate
over requests, so it needs at least 10^4 requests to be measured. Every request where the GPU and
the oracle differ must be flagged by the oracle (a uniform within 1e-5 of its acceptance ratio, or
u*S within 1e-5*S of a CDF boundary), and differing requests must stay below 1e-4 of all requests.
Tiny and mid pool 10^4 requests here; the large workload pools 2048 here (its inputs take seconds
per seed to generate) and ``bench.py --pooled-parity tiny,mid,large,ragged`` runs every workload at
10^4 or more."""
import numpy as np
import pytest

import inputgen
import oracle
from _parity import FLAG, device_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    import torch

    import rejection_sampling_verify_spec_amd as m
    assert torch.cuda.is_available(), "GPU tests need a visible GPU"
    return m


@pytest.mark.parametrize("name,seeds", [("tiny", 1250), ("mid", 157), ("large", 8)])
def test_pooled(sv, name, seeds):
    import torch
    req = mism = unflagged = flagged = 0
    for k in range(seeds):
        d = inputgen.make(name, seed=1000 + k)
        t = device_inputs(d)
        out, na = sv.verify_chain(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"],
                                  t["temperature"])
        torch.cuda.synchronize()
        out, na = out.cpu().numpy(), na.cpu().numpy()
        ref = oracle.verify_chain(d["target"], d["draft"], d["draft_tokens"], d["u_accept"], d["u_sample"],
                                  d["temperature"])
        m = (na != ref["num_accepted"]) | (out != ref["out_tokens"]).any(axis=1)
        f = (ref["acc_margin"] < FLAG) | (ref["cdf_margin"] < FLAG)
        req += na.shape[0]
        mism += int(m.sum())
        unflagged += int((m & ~f).sum())
        flagged += int(f.sum())
        if k % max(1, seeds // 5) == 0:
            print(f"[pooled {name}] seed {1000 + k}: {req} requests, {mism} mismatches", flush=True)
    print(f"[pooled {name}] {req} requests, {mism} mismatches ({unflagged} unflagged), "
          f"flagged {flagged / req:.4f}", flush=True)
    assert unflagged == 0
    assert mism < 1e-4 * req
    assert (np.asarray(req) >= (10_000 if name != "large" else 2048))
