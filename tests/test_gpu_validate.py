"""GPU parity of validate_page_tags: verdicts must be bit-exact against the
oracle and equal to the mismatches injected by construction."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import log

pytestmark = pytest.mark.gpu


def _run(gpu, tags, bt, exp, lens, S):
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(
        np.int32 if a.dtype in (np.uint32, np.int32) else a.dtype)).cuda()
    ver = torch.full((bt.shape[0],), 12345, dtype=torch.int32, device="cuda")
    gpu.validate_page_tags(d(tags), d(bt), d(exp), d(lens), ver, page_size=S)
    torch.cuda.synchronize()
    return ver.cpu().numpy()


@pytest.mark.parametrize("cid", [1, 5])
def test_workload_verdicts(gpu, cid):
    log(f"validate workload {cid}")
    b = synth.make_batch(cid)
    S = b.cfg.page_size
    got = _run(gpu, b.page_tags, b.block_table, b.expected_tags, b.seq_lens, S)
    want = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags, b.seq_lens, S)
    assert np.array_equal(got, want)
    inj = np.zeros(b.B, np.int32)
    for s, j in b.injected:
        inj[s] = j + 1 if inj[s] == 0 else min(inj[s], j + 1)
    assert np.array_equal(got, inj)
    assert (got != 0).sum() >= 1


def test_edge_cases(gpu):
    log("validate edge cases")
    rng = np.random.default_rng(3)
    B, S, P, mb = 1003, 16, 5000, 300
    lens = rng.integers(0, mb * S + 1, B).astype(np.int32)
    tags = rng.integers(0, 2 ** 32, P, dtype=np.uint64).astype(np.uint32)
    bt = rng.integers(0, P, (B, mb)).astype(np.int32)
    exp = tags[bt]
    # faults at random blocks (inside and outside the valid range)
    for s in rng.choice(B, 200, replace=False):
        j = int(rng.integers(0, mb))
        kind = int(rng.integers(0, 4))
        if kind == 0:
            exp[s, j] ^= np.uint32(1 << int(rng.integers(0, 32)))
        elif kind == 1:
            bt[s, j] = P + int(rng.integers(0, 10))
        elif kind == 2:
            bt[s, j] = -1 - int(rng.integers(0, 10))
        else:
            bt[s, j] = (bt[s, j] + 1) % P
    lens[0] = 0
    lens[1] = -5
    lens[2] = mb * S + 1
    lens[3] = mb * S
    got = _run(gpu, tags, bt, exp, lens, S)
    want = oracle.validate_page_tags(tags, bt, exp, lens, S)
    assert np.array_equal(got, want)
    assert got[1] == -1 and got[2] == -1
    assert (got > 0).sum() > 50
