"""GPU-test helpers: oracle-side caches for chosen sequences of a workload,
and the attention tolerance check. The oracle never sees anything the GPU
produced: it quantises the same seeded bf16 inputs itself."""
from __future__ import annotations

import sys

import numpy as np

from oracle.harness import (oracle_attn_subset, oracle_subset,  # noqa: F401
                            oracle_write_threaded, threads)

# Attention parity bar: max |gpu - oracle| <= 2e-3 and
# ||gpu - oracle||_2 / ||oracle||_2 <= 1e-3 over the compared rows.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def attn_errors(got: np.ndarray, ref: np.ndarray):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / den) if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_attn_close(got, ref, what=""):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert np.array_equal(np.isnan(got), np.isnan(ref)), f"{what}: NaN pattern differs"
    ok = ~np.isnan(ref)
    max_abs, rel = attn_errors(got[ok], ref[ok])
    assert max_abs <= MAX_ABS and rel <= REL_L2, f"{what}: max_abs={max_abs:.3e} rel_l2={rel:.3e}"
    return max_abs, rel


def gpu_pages(cache_t, pages, page_elems):
    """Host copy of the given physical pages of a flat GPU cache tensor."""
    import torch
    idx = torch.as_tensor(np.asarray(pages, np.int64), device=cache_t.device)
    return cache_t.view(-1, page_elems).index_select(0, idx).cpu().numpy()
