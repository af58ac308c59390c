"""The Python binding has no CPU path (no GPU needed): without the HIP library the
package does not import, and host tensors are refused before any library call."""
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_import_fails_without_the_library():
    env = dict(os.environ, SPECVERIFY_LIB=os.path.join(ROOT, "no_such_dir", "libspecverify.so"))
    code = "import rejection_sampling_verify_spec_amd"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode != 0
    assert "ImportError" in r.stderr and "not built" in r.stderr


def test_host_tensors_are_refused():
    import torch

    import inputgen
    import rejection_sampling_verify_spec_amd as sv
    d = inputgen.chain_inputs(2, 2, 64, seed=1, dtype="f32")
    t = {k: torch.from_numpy(np.ascontiguousarray(v)) for k, v in d.items() if isinstance(v, np.ndarray)}
    with pytest.raises(ValueError, match="device tensor"):
        sv.verify_chain(t["target"], t["draft"], t["draft_tokens"], t["u_accept"], t["u_sample"], t["temperature"])
    rows = torch.from_numpy(inputgen.logit_rows(2, 64, np.arange(3, dtype=np.int64), dtype="f32"))
    with pytest.raises(ValueError, match="device tensor"):
        sv.sample_rows(rows, torch.ones(3), torch.full((3,), 0.5))
