"""The LDS read-bandwidth probe behind the benchmark's LDS roofline: every
thread's output word equals the fold of the two words its last iteration read,
computed here from the buffer's closed form, so the reads the probe times are
the reads it was written to make."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def expected_words(blocks: int, iters: int) -> np.ndarray:
    """Word i of the 64 KiB buffer is (i, 3i+1, 5i+2, 7i+3).  Thread t starts
    at t mod 2048 and moves 64 words per iteration (mod 2048); its output is
    the XOR of the four lanes of word[s] ^ word[s + 1792], s its last start."""
    tid = np.arange(1024, dtype=np.uint64)
    s = (tid % 2048 + 64 * (iters - 1)) % 2048

    def fold(i):
        return i ^ (3 * i + 1) ^ (5 * i + 2) ^ (7 * i + 3)

    w = (fold(s) ^ fold(s + 1792)) & 0xFFFFFFFF
    return np.tile(w.astype(np.uint32), blocks)


@pytest.mark.parametrize("blocks,iters", [(1, 1), (3, 33), (512, 64)])
def test_lds_probe_reads_what_it_claims(blocks, iters):
    import torch
    from experiment_network_simulation_amd.sim import lds_probe
    out = torch.full((blocks * 1024,), -1, dtype=torch.int32, device="cuda:0")
    nbytes = lds_probe(out, blocks, iters)
    torch.cuda.synchronize()
    assert nbytes == blocks * 1024 * iters * 128
    got = out.cpu().numpy().view(np.uint32)
    assert np.array_equal(got, expected_words(blocks, iters))
