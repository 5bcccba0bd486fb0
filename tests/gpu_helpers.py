"""GPU-test helpers: oracle-side caches for chosen sequences of a workload,
and the attention tolerance check. The oracle never sees anything the GPU
produced: it quantises the same seeded bf16 inputs itself."""
from __future__ import annotations

import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

# Attention parity bar: max |gpu - oracle| <= 2e-3 and
# ||gpu - oracle||_2 / ||oracle||_2 <= 1e-3 over the compared rows.
MAX_ABS = 2e-3
REL_L2 = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def threads() -> int:
    return min(16, os.cpu_count() or 1)


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


def oracle_write_threaded(fn, k, v, slots, nthreads=None, **kw):
    """Run an oracle kv_write over token slices in parallel threads (the
    slices touch disjoint slots)."""
    T = k.shape[0]
    n = nthreads or threads()
    step = max(1, -(-T // n))
    parts = [(i, min(T, i + step)) for i in range(0, T, step)]

    def run(p):
        a, b = p
        fn(k[a:b], None if v is None else v[a:b], slots[a:b], **kw)

    with ThreadPoolExecutor(len(parts)) as ex:
        list(ex.map(run, parts))


def oracle_subset(batch: synth.Batch, data, seqs, kv_dtype, host_scales, poison=True):
    """Oracle caches holding only sequences `seqs`, in a compact pool whose
    page j is the j-th page those sequences use (block tables remapped;
    attention is invariant to the physical placement). Returns a dict with
    the caches, compact block table, lens, q rows and the list of original
    page ids in compact order."""
    cfg = batch.cfg
    S, hkv, dk, dv = cfg.page_size, cfg.num_kv_heads, cfg.head_dim_qk, cfg.head_dim_v
    pages = []
    for s in seqs:
        n = -(-int(batch.seq_lens[s]) // S)
        pages.extend(int(p) for p in batch.block_table[s, :n])
    P = max(len(pages), 1)
    remap = {p: j for j, p in enumerate(pages)}
    bt = np.full((len(seqs), batch.max_blocks), -1, np.int32)
    for i, s in enumerate(seqs):
        n = -(-int(batch.seq_lens[s]) // S)
        bt[i, :n] = [remap[int(p)] for p in batch.block_table[s, :n]]
    fp8 = kv_dtype == synth.KV_FP8
    dt = np.uint8 if fp8 else np.uint16
    fill = synth.poison_value(kv_dtype) if poison else 0
    kc = np.full(P * hkv * S * dk, fill, dt)
    vc = None if cfg.v_in_k else np.full(P * hkv * S * dv, fill, dt)
    ts = np.full(P * S, np.nan, np.float32) if (fp8 and cfg.v_in_k) else None
    for i, s in enumerate(seqs):
        l = int(batch.seq_lens[s])
        if l == 0:
            continue
        k, v = data[s]
        t = np.arange(l, dtype=np.int64)
        slots = bt[i, t // S].astype(np.int64) * S + t % S
        if fp8:
            mode = synth.SCALE_PER_TOKEN if cfg.v_in_k else synth.SCALE_PER_HEAD
            oracle_write_threaded(
                oracle.kv_write_fp8, k, v, slots, page_size=S, num_pages=P, scale_mode=mode,
                k_scale=None if cfg.v_in_k else host_scales[0],
                v_scale=None if cfg.v_in_k else host_scales[1], token_scale=ts,
                k_cache=kc, v_cache=vc)
        else:
            oracle_write_threaded(oracle.kv_write_bf16, k, v, slots, page_size=S,
                                  num_pages=P, k_cache=kc, v_cache=vc)
    return dict(kc=kc, vc=vc, ts=ts, bt=bt, P=P, pages=pages,
                lens=batch.seq_lens[list(seqs)].astype(np.int32),
                q=batch.q[list(seqs)])


def oracle_attn_subset(batch: synth.Batch, sub, kv_dtype, host_scales, verdict=None,
                       rows=None):
    cfg = batch.cfg
    fp8 = kv_dtype == synth.KV_FP8
    if fp8 and cfg.v_in_k:
        mode, ks, vs = synth.SCALE_PER_TOKEN, sub["ts"], None
    elif fp8:
        mode, ks, vs = synth.SCALE_PER_HEAD, host_scales[0], host_scales[1]
    else:
        mode, ks, vs = synth.SCALE_NONE, None, None
    return oracle.paged_decode_attn(
        sub["q"], sub["kc"], sub["vc"], ks, vs, sub["bt"], sub["lens"],
        num_kv_heads=cfg.num_kv_heads, head_dim_v=cfg.head_dim_v, page_size=cfg.page_size,
        num_pages=sub["P"], kv_dtype=kv_dtype, scale_mode=mode, v_in_k=cfg.v_in_k,
        sm_scale=cfg.sm_scale, verdict=verdict, rows=rows, num_threads=threads())


def gpu_pages(cache_t, pages, page_elems):
    """Host copy of the given physical pages of a flat GPU cache tensor."""
    import torch
    idx = torch.as_tensor(np.asarray(pages, np.int64), device=cache_t.device)
    return cache_t.view(-1, page_elems).index_select(0, idx).cpu().numpy()
