"""The read-ceiling probe (a measurement aid): every 16-byte vector of the
buffer is read, checked through the per-wave folded words against the same
fold computed on the host."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

VEC_PER_BLOCK, THREADS, UNROLL = 2048, 256, 4


def host_fold(words):
    vec = words.reshape(-1, 4)
    nvec = vec.shape[0]
    nblk = (nvec + VEC_PER_BLOCK - 1) // VEC_PER_BLOCK
    out = np.zeros(nblk * 4, np.uint32)
    per_vec = vec[:, 0] ^ vec[:, 1] ^ vec[:, 2] ^ vec[:, 3]
    for blk in range(nblk):
        for tid in range(THREADS):
            acc = np.uint32(0)
            for k0 in range(tid, VEC_PER_BLOCK, THREADS * UNROLL):
                for u in range(UNROLL):
                    i = blk * VEC_PER_BLOCK + k0 + u * THREADS
                    if i < nvec:
                        acc ^= per_vec[i]
            out[blk * 4 + tid // 64] ^= acc
    return out


def test_read_probe_reads_every_vector():
    import torch

    import rejection_sampling_verify_spec_amd as sv
    rng = np.random.default_rng(3)
    words = rng.integers(0, 2 ** 32, size=(2 * VEC_PER_BLOCK + 37) * 4, dtype=np.uint64).astype(np.uint32)
    t = torch.from_numpy(words.view(np.int32)).cuda()
    out = sv.read_probe(t)
    torch.cuda.synchronize()
    assert out.numel() == sv.spec_read_probe_words(words.nbytes)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), host_fold(words))
