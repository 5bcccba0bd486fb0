"""Full-size GPU parity on every output row and every cache byte: the 32 x
8192 (BF16 and FP8), 64 x 8192 (FP8, K outliers, split 512), latent (64
sequences of U[1024, 32768] tokens, 128 query heads, per-token scales) and
full-pool (256 lognormal sequences, churned pool, injected tag mismatches)
workloads, launched exactly as the benchmark launches them (its default
workspace and split, one whole step: kv write of the newest token, tag
check, attention).

The oracle quantises the same seeded bf16 inputs of every sequence into its
own full-size pool at the same physical page ids, so the device caches are
compared byte for byte over the whole pool (unused pages must still hold the
poison both sides start from), the verdicts bit for bit, and every
non-aborted output row within the attention tolerance (max |diff| <= 2e-3,
rel-L2 <= 1e-3 over the compared rows); aborted rows must be zero.
"""
import gc

import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_attn_close, log, threads
from oracle.harness import oracle_attn_full, oracle_full_cache

pytestmark = pytest.mark.gpu

_DATA = {}     # per-sequence bf16 inputs of one workload at a time
_RUNS = {}     # results of one (workload, dtype) at a time


def _data(cid, b):
    if cid not in _DATA:
        _DATA.clear()
        gc.collect()
        log(f"  generating workload {cid} inputs")
        _DATA[cid] = synth.map_seqs(lambda s: b.kv(s), list(range(b.B)), threads())
    return _DATA[cid]


def _run(cid, kv_dtype):
    """Device step + oracle caches for one workload; cached for the tests of
    that workload (the compare of rows is split over several tests where the
    oracle needs long)."""
    key = (cid, kv_dtype)
    if key in _RUNS:
        return _RUNS[key]
    _RUNS.clear()
    gc.collect()
    from synth import device as workload
    b = synth.make_batch(cid)
    data = _data(cid, b)
    log(f"  workload {cid}: device caches (dtype {kv_dtype}) and one step")
    db = workload.build(b, kv_dtype, data=data)
    db.alloc_workspace()
    db.step(use_verdict=True)
    torch.cuda.synchronize()
    verdict = db.verdict.cpu().numpy()
    got = db.out.cpu().numpy()
    gk = db.k_cache.cpu().numpy()
    gv = None if db.v_cache is None else db.v_cache.cpu().numpy()
    gts = db.k_scale.cpu().numpy() if (b.cfg.v_in_k and kv_dtype == synth.KV_FP8) else None
    host_scales = db.host_scales
    del db
    torch.cuda.empty_cache()
    log(f"  workload {cid}: oracle caches of all {b.B} sequences")
    kc, vc, ts = oracle_full_cache(b, data, kv_dtype, host_scales)
    elt = np.uint8 if kv_dtype == synth.KV_FP8 else np.uint16
    assert np.array_equal(gk.view(elt), kc), "K cache differs from the oracle"
    if vc is not None:
        assert np.array_equal(gv.view(elt), vc), "V cache differs from the oracle"
    if ts is not None:
        assert np.array_equal(gts.view(np.uint32), ts.view(np.uint32)), \
            "token scales differ from the oracle"
    del gk, gv, gts
    want_verdict = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags,
                                             b.seq_lens, b.cfg.page_size)
    assert np.array_equal(verdict, want_verdict), "verdicts differ from the oracle"
    _RUNS[key] = (b, got, want_verdict, kc, vc, ts, host_scales)
    return _RUNS[key]


def _compare(cid, kv_dtype, seqs=None):
    b, got, verdict, kc, vc, ts, host_scales = _run(cid, kv_dtype)
    seqs = list(range(b.B)) if seqs is None else list(seqs)
    log(f"  workload {cid}: oracle attention, {len(seqs)} sequences x "
        f"{b.cfg.num_q_heads} heads")
    ref = oracle_attn_full(b, kc, vc, ts, kv_dtype, host_scales, verdict, seqs)
    g = got[seqs]
    aborted = verdict[seqs] != 0
    assert np.all(g[aborted] == 0), "aborted rows must be zero"
    assert np.all(ref[aborted] == 0)
    mx, rel = assert_attn_close(g[~aborted], ref[~aborted],
                                f"workload {cid} dtype {kv_dtype} seqs {seqs[0]}..{seqs[-1]}")
    log(f"  workload {cid}: {int((~aborted).sum())} sequences compared, "
        f"max_abs {mx:.3e} rel_l2 {rel:.3e}")
    return b, verdict


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
def test_workload2_all_rows(gpu, kv_dtype):
    log(f"workload 2 full size, dtype {kv_dtype}")
    b, verdict = _compare(2, kv_dtype)
    assert np.all(verdict == 0)


def test_workload3_all_rows(gpu):
    log("workload 3 full size")
    b, verdict = _compare(3, synth.KV_FP8)
    assert np.all(verdict == 0)


def test_workload3_no_op_tracker_same_bits(gpu):
    """The no-op tracker (no check, NULL verdict) gives the same bits as an
    all-clear verdict on the 64 x 8192 workload."""
    from synth import device as workload
    b = synth.make_batch(3)
    data = _data(3, b)
    db = workload.build(b, synth.KV_FP8, data=data)
    db.alloc_workspace()
    db.step(use_verdict=True)
    torch.cuda.synchronize()
    out1 = db.out.clone()
    db.attend(use_verdict=False)
    torch.cuda.synchronize()
    assert torch.equal(out1, db.out)


def test_workload5_all_rows(gpu):
    log("workload 5 full size")
    b, verdict = _compare(5, synth.KV_FP8)
    inj = sorted({s for s, _ in b.injected})
    assert len(inj) >= 1 and (verdict != 0).sum() == len(inj)
    assert sorted(np.nonzero(verdict)[0].tolist()) == inj


@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_workload4_all_rows(gpu, part):
    """Latent workload on the matrix-core path; the oracle's rows are split
    over four tests of 16 sequences (the 128-head fp64 oracle is the slow
    part)."""
    log(f"workload 4 full size, sequences {16 * part}..{16 * part + 15}")
    b, verdict = _compare(4, synth.KV_FP8, range(16 * part, 16 * part + 16))
    assert np.all(verdict == 0)


@pytest.mark.parametrize("kv_dtype", [synth.KV_BF16, synth.KV_FP8])
@pytest.mark.parametrize("B", [1, 8])
def test_concurrency_sweep_shapes(gpu, B, kv_dtype):
    """The smaller batches of the concurrency sweep (B sequences of 8192
    tokens, the 64 x 8192 workload's heads and outliers, automatic split-K:
    128-token chunks for 8 sequences, 64 for one), launched as bench.py
    --sweep launches them; every sequence compared."""
    from oracle.harness import oracle_attn_subset, oracle_subset
    from synth import device as workload
    _RUNS.clear()
    _DATA.clear()
    gc.collect()
    log(f"sweep shape B={B}, dtype {kv_dtype}")
    b = synth.make_batch(3, lens=[8192] * B)
    data = synth.map_seqs(lambda s: b.kv(s), list(range(B)), threads())
    db = workload.build(b, kv_dtype, data=data)
    db.alloc_workspace(split_tokens=0)
    db.step(use_verdict=True)
    torch.cuda.synchronize()
    verdict = db.verdict.cpu().numpy()
    assert np.all(verdict == 0)
    got = db.out.cpu().numpy()
    seqs = list(range(B))
    sub = oracle_subset(b, data, seqs, kv_dtype, db.host_scales)
    ref = oracle_attn_subset(b, sub, kv_dtype, db.host_scales, verdict=verdict)
    assert_attn_close(got, ref, f"sweep B={B} dtype {kv_dtype}")
