"""Oracle-side helpers for the synthetic workloads: oracle caches holding
chosen sequences of a workload, quantised by the oracle itself from the same
seeded bf16 inputs, and the oracle's attention over them.

TEST INFRASTRUCTURE ONLY, like the rest of this package: used by ``tests/``,
the smoke check and the CPU-baseline leg of ``bench.py``. Nothing here ever
sees an output of the GPU path.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth


def threads() -> int:
    return min(16, os.cpu_count() or 1)


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


def oracle_full_cache(batch: synth.Batch, data, kv_dtype, host_scales, poison=True):
    """Oracle caches of a whole workload at its own physical page ids: a pool
    of batch.num_pages pages filled with the poison value (the value the
    device caches of the same workload are filled with before their context
    is written), then every context token of every sequence quantised (or
    copied, BF16) into its slot by the oracle's kv_write. Returns (kc, vc,
    ts): flat caches in the library's format and, for per-token scaling, the
    token scales (NaN where no token was written)."""
    cfg = batch.cfg
    S, P = cfg.page_size, batch.num_pages
    hkv, dk, dv = cfg.num_kv_heads, cfg.head_dim_qk, cfg.head_dim_v
    fp8 = kv_dtype == synth.KV_FP8
    dt = np.uint8 if fp8 else np.uint16
    fill = synth.poison_value(kv_dtype) if poison else 0
    kc = np.full(P * hkv * S * dk, fill, dt)
    vc = None if cfg.v_in_k else np.full(P * hkv * S * dv, fill, dt)
    ts = np.full(P * S, np.nan, np.float32) if (fp8 and cfg.v_in_k) else None

    def one(s):
        l = int(batch.seq_lens[s])
        if l == 0:
            return
        k, v = data[s]
        slots = batch.slots(s, np.arange(l)).astype(np.int64)
        if fp8:
            oracle.kv_write_fp8(
                k, v, slots, S, P,
                synth.SCALE_PER_TOKEN if cfg.v_in_k else synth.SCALE_PER_HEAD,
                None if cfg.v_in_k else host_scales[0],
                None if cfg.v_in_k else host_scales[1], ts, kc, vc)
        else:
            oracle.kv_write_bf16(k, v, slots, S, P, kc, vc)

    # sequences own disjoint pages, so their writes never touch one byte twice
    with ThreadPoolExecutor(threads()) as ex:
        list(ex.map(one, range(batch.B)))
    return kc, vc, ts


def oracle_attn_full(batch: synth.Batch, kc, vc, ts, kv_dtype, host_scales, verdict,
                     seqs=None):
    """Oracle attention over the full-pool caches of oracle_full_cache, for
    every query head of the sequences `seqs` (all when None). Returns
    [len(seqs), Hq, Dv] fp32 rows (rows of other sequences are not
    computed)."""
    cfg = batch.cfg
    fp8 = kv_dtype == synth.KV_FP8
    if fp8 and cfg.v_in_k:
        mode, ks, vs = synth.SCALE_PER_TOKEN, ts, None
    elif fp8:
        mode, ks, vs = synth.SCALE_PER_HEAD, host_scales[0], host_scales[1]
    else:
        mode, ks, vs = synth.SCALE_NONE, None, None
    seqs = list(range(batch.B)) if seqs is None else list(seqs)
    rows = np.array([(s, h) for s in seqs for h in range(cfg.num_q_heads)], np.int32)
    out = oracle.paged_decode_attn(
        batch.q, kc, vc, ks, vs, batch.block_table, batch.seq_lens,
        num_kv_heads=cfg.num_kv_heads, head_dim_v=cfg.head_dim_v, page_size=cfg.page_size,
        num_pages=batch.num_pages, kv_dtype=kv_dtype, scale_mode=mode, v_in_k=cfg.v_in_k,
        sm_scale=cfg.sm_scale, verdict=verdict, rows=rows, num_threads=threads())
    return out[seqs]
