#!/usr/bin/env python3
"""Benchmark of one decode step of the FP8 paged decode-attention path on one
MI355X, on the 64 sequences x 8192-token workload (64 query / 8 kv heads,
head dim 128, pages of 16 tokens, FP8 e4m3 cache with per-head scales and 6 of
128 K channels per kv head scaled by 20, split-K chunks of 512 tokens).

A step = the kv write of every sequence's newest token and the page-tag
check in one launch (kv_write_check) + paged_decode_attn (split-K partials +
combine), all on one stream with the inputs resident in HBM; the same step
with kv_write_fp8 and validate_page_tags as two launches is timed beside it.
The same step is timed with a BF16 cache built from the same bf16 inputs,
for the FP8/BF16 ratio.

Prints one JSON line. `value` is algorithmic KV bytes per step / step time
(GB/s). `roofline` rates the attention call (partial + combine kernels),
timed with HIP events on the launch stream. `cpu_baseline` times the oracle
on a bounded sample of the same workload on the host cores.

    python bench.py [--steps K] [--warmup W] [--passes N] [--gpus 1]
                    [--schedule serial|overlap] [--no-cpu-baseline] [--no-extra]

Every timed figure is the median over N interleaved passes of exactly K
calls between two HIP events on the launch stream (FP8 and BF16 steps, the
attention calls alone, and the no-op-tracker step alternate within each
pass), after W warm-up steps. The tag check's share of the step is the
median over the passes of the ratio of the step with the check to the step
with the no-op tracker timed right after it. Extra keys: the latent workload's attention
call against the matrix-core peak, the full-pool workload's step with the
tag check's share, the BF16 -> FP8 page transcode, the INT4 GEMV.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = ("decode-attn KV GB/s (% HBM peak) + seq-steps/s, FP8 vs BF16 KV, 64×8k ctx")
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, AMD specification
MFMA_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 / f16 matrix peak, AMD specification
LATENT_SETTLE_CALLS = 120       # untimed latent calls before its passes (clock settling)
WORKLOAD_ID = 3
DEFAULT_SCHEDULE = "serial"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_64x8k.txt")
KERNEL_SOURCE = os.path.join(ROOT, "decode_attention_fp8_write_amd", "csrc", "decode_attn.hip")


def code_hash(path):
    """sha256 of a C++/HIP source with its comments and blank lines removed,
    so that a comment edit does not invalidate the counters recorded for the
    code (string literals in these sources hold no comment markers)."""
    import hashlib
    import re
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in text.splitlines()]
    return hashlib.sha256("\n".join(ln for ln in lines if ln).encode()).hexdigest()


def measured_traffic():
    """HBM bytes per attention call (partial + combine) from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE runs, scaled by the copy-kernel
    calibration; None when the kernel code changed since they were taken."""
    try:
        fields = {}
        for line in open(TRAFFIC_FILE):
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                fields[k.strip()] = v.strip()
        if fields.get("decode_attn.hip code sha256") != code_hash(KERNEL_SOURCE):
            return None
        return int(fields["hbm bytes per attention call"])
    except (OSError, KeyError, ValueError):
        return None


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def median(xs):
    xs = sorted(xs)
    n = len(xs)
    return xs[n // 2] if n % 2 else 0.5 * (xs[n // 2 - 1] + xs[n // 2])


def timed_pass(fn, steps, torch):
    """Mean milliseconds of one call of fn over exactly `steps` calls between
    two HIP events on the current (launch) stream, synchronised on both
    sides."""
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        fn()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / steps


def interleaved_passes(fns, steps, passes, torch):
    """`passes` rounds; each round times every named function once over
    exactly `steps` calls (timed_pass), in the given order, so that clock
    and temperature drift reach every function alike. Returns name -> list
    of per-pass milliseconds per call."""
    out = {name: [] for name in fns}
    for _ in range(passes):
        for name, fn in fns.items():
            out[name].append(timed_pass(fn, steps, torch))
    return out


def breakdown(db, steps, torch):
    """One pass with an event between the calls of every step, all on one
    stream: the mean duration of the kv write, the tag check and the
    attention call. The events cost time of their own, so the step time
    never comes from here."""
    evs = []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
        e[0].record()
        db.write_step()
        e[1].record()
        db.validate()
        e[2].record()
        db.attend()
        e[3].record()
        evs.append(e)
    torch.cuda.synchronize()
    # the same with the write and the check in one launch (kv_write_check)
    fev = []
    for _ in range(steps):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        db.write_check()
        e[1].record()
        db.attend()
        e[2].record()
        fev.append(e)
    torch.cuda.synchronize()
    mean = lambda xs: sum(xs) / len(xs)
    return dict(kv_write_ms=mean([e[0].elapsed_time(e[1]) for e in evs]),
                validate_ms=mean([e[1].elapsed_time(e[2]) for e in evs]),
                attn_ms_with_events=mean([e[2].elapsed_time(e[3]) for e in evs]),
                step_ms_with_call_events=mean([e[0].elapsed_time(e[3]) for e in evs]),
                write_check_ms=mean([e[0].elapsed_time(e[1]) for e in fev]),
                step_ms_fused_with_call_events=mean([e[0].elapsed_time(e[2]) for e in fev]))


def pool_cycles(pool, seconds):
    """Pages per second of alloc + free of the 512 pages of one 8192-token
    sequence (page 16) per cycle."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        pages = pool.alloc(512)[0]
        pool.free(pages)
        n += 512
    return n / (time.perf_counter() - t0)


def time_page_pool(pda, np, seconds=0.3):
    """Host page pool throughput (libpda.so's pda_pool_*), tracking on and
    off, on a 32768-page pool (the 64 x 8192 workload's pool)."""
    P = 32768
    order = np.random.default_rng(1).permutation(P)
    res = {}
    for name, track in (("tags", True), ("no_op", False)):
        pool = pda.PagePool(P, initial_order=order, track_tags=track)
        res[f"native_{name}_pages_per_s"] = pool_cycles(pool, seconds)
        pool.close()
    return res


def read_ceiling(torch, pda, reps=10):
    """Measured HBM read ceilings (pda_hbm_read_probe over a 4 GiB buffer):
    one streaming pass, and 2 KB chunks in scrambled order (the per-page,
    per-kv-head granule of the FP8 cache at page 16)."""
    buf = torch.ones(1 << 30, dtype=torch.int32, device="cuda")
    sink = torch.zeros(pda.hbm_read_probe_sink_words(), dtype=torch.int32, device="cuda")
    out = {}
    for name, chunk in (("streaming_GBps", 0), ("random_2KB_GBps", 2048)):
        for _ in range(2):
            pda.hbm_read_probe(buf, chunk, sink)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            pda.hbm_read_probe(buf, chunk, sink)
        b.record()
        torch.cuda.synchronize()
        out[name] = (4 << 30) / (a.elapsed_time(b) / reps * 1e-3) / 1e9
    del buf, sink
    torch.cuda.empty_cache()
    log(f"measured read ceilings: {out}")
    return out


def time_transcode(bf, fp8, args, torch, np, pda, reps=50):
    """kv_transcode_bf16_to_fp8 of every page of the BF16 pool into a fresh
    FP8 pool of the same size through a seeded permutation, timed with HIP
    events on the launch stream over `reps` calls after a few warm-up calls.
    Algorithmic bytes: BF16 K+V read, FP8 K+V written, 12 bytes of page
    arrays per page."""
    cfg = bf.cfg
    S, P, hkv = cfg.page_size, bf.batch.num_pages, cfg.num_kv_heads
    dk, dv = cfg.head_dim_qk, cfg.head_dim_v
    rng = np.random.default_rng(77)
    src = torch.arange(P, dtype=torch.int32, device="cuda")
    dst = torch.from_numpy(rng.permutation(P).astype(np.int32)).cuda()
    valid = torch.full((P,), S, dtype=torch.int32, device="cuda")
    kd = torch.empty(P * hkv * S * dk, dtype=torch.uint8, device="cuda")
    vd = torch.empty(P * hkv * S * dv, dtype=torch.uint8, device="cuda")

    def call():
        pda.kv_transcode_bf16_to_fp8(
            bf.k_cache, bf.v_cache, src, dst, valid, kd, vd, num_kv_heads=hkv, head_dim_k=dk,
            head_dim_v=dv, page_size=S, src_num_pages=P, dst_num_pages=P,
            scale_mode=pda.SCALE_PER_HEAD, k_scale=fp8.k_scale, v_scale=fp8.v_scale)

    for _ in range(5):
        call()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        call()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    nbytes = P * hkv * S * (dk + dv) * (2 + 1) + 12 * P
    gbps = nbytes / (ms * 1e-3) / 1e9
    log(f"transcode of {P} pages: {ms:.4f} ms, {gbps:.0f} GB/s")
    return {"pages": P, "ms": ms, "algorithmic_bytes_per_launch": nbytes,
            "roofline": {"kernel": "kv_transcode_head_kernel", "bound": "hbm",
                         "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                         "frac": gbps / HBM_PEAK_GBPS}}


def time_int4(torch, pda, n=8192, k=8192, batches=(1, 8, 16, 32, 64), nmat=16, reps=64):
    """int4_gemv_bf16 on an n x k weight matrix, cycling through `nmat`
    independent matrices (more bytes than the chip's caches hold, so every
    call streams its weights from HBM), timed with HIP events on the launch
    stream; beside it the same product with dense bf16 weights through
    torch's linear (hipBLASLt), the format the INT4 weights replace.
    Algorithmic bytes per call: codes n*k/2, scales n*k/128*2, x m*k*2,
    y m*n*4."""
    gen = torch.Generator(device="cuda").manual_seed(11)
    ws = [torch.randint(-2 ** 31, 2 ** 31 - 1, (n, k // 8), generator=gen, dtype=torch.int32,
                        device="cuda") for _ in range(nmat)]
    ss = [((torch.rand((n, k // 128), generator=gen, device="cuda") - 0.5) * 0.1)
          .to(torch.bfloat16) for _ in range(nmat)]
    out = {"shape": {"n": n, "k": k}, "matrices_cycled": nmat, "by_tokens": {}}
    for m in batches:
        x = torch.randn((m, k), generator=gen, device="cuda").to(torch.bfloat16)
        y = torch.empty((m, n), dtype=torch.float32, device="cuda")

        def call(i):
            pda.int4_gemv_bf16(x, ws[i % nmat], ss[i % nmat], y)

        for i in range(8):
            call(i)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            call(i)
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        nbytes = n * k // 2 + n * (k // 128) * 2 + m * k * 2 + m * n * 4
        gbps = nbytes / (ms * 1e-3) / 1e9
        out["by_tokens"][str(m)] = {
            "us": ms * 1e3, "algorithmic_bytes": nbytes, "GBps": gbps,
            "frac_hbm": gbps / HBM_PEAK_GBPS, "TFLOPs": 2.0 * m * n * k / (ms * 1e-3) / 1e12}
        log(f"int4 gemv m={m}: {ms * 1e3:.2f} us, {gbps:.0f} GB/s")
    # dense bf16 weights of the same shape, same cycling
    wb = [torch.randn((n, k), generator=gen, device="cuda").to(torch.bfloat16)
          for _ in range(nmat)]
    for m in batches:
        x = torch.randn((m, k), generator=gen, device="cuda").to(torch.bfloat16)
        for i in range(8):
            torch.nn.functional.linear(x, wb[i % nmat])
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(reps):
            torch.nn.functional.linear(x, wb[i % nmat])
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        r = out["by_tokens"][str(m)]
        r["bf16_dense_us"] = ms * 1e3
        r["speedup_vs_bf16_dense"] = ms * 1e3 / r["us"]
        log(f"bf16 dense linear m={m}: {ms * 1e3:.2f} us")
    r1 = out["by_tokens"][str(batches[0])]
    out["roofline"] = {"kernel": "int4_gemv_kernel", "tokens": batches[0], "bound": "hbm",
                       "achieved": r1["GBps"], "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                       "frac": r1["frac_hbm"]}
    del ws, ss, wb
    torch.cuda.empty_cache()
    return out


def int4_oracle_rate(np, synth, n=8192, k=8192, cols=2048):
    """The oracle's INT4 GEMV for one token on `cols` output columns of an
    n x k matrix, scaled to whole GEMVs per second."""
    import oracle
    rng = np.random.default_rng(3)
    x = synth.bf16_from_f32(rng.standard_normal((1, k)).astype(np.float32))
    w = rng.integers(0, 1 << 32, (n, k // 8), dtype=np.uint64).astype(np.uint32)
    s = synth.bf16_from_f32(rng.uniform(-0.05, 0.05, (n, k // 128)).astype(np.float32))
    t0 = time.perf_counter()
    oracle.int4_gemv(x, w, s, cols=np.arange(cols))
    t = time.perf_counter() - t0
    return {"gemv_per_s": cols / n / t, "cores": 1,
            "sample": f"{cols} of {n} output columns, 1 token, k {k}; {t:.2f} s"}


def cpu_baseline(batch, data, host_scales, target_s=12.0):
    """The oracle (fp64, plain loops, all host threads) running the same
    step on whole sequences of the workload: kv write of the newest token,
    tag validation, attention for every query head."""
    import numpy as np

    import oracle
    import synth
    from oracle.harness import oracle_subset

    cfg = batch.cfg
    nthreads = os.cpu_count() or 1

    def run(seqs, sub):
        t0 = time.perf_counter()
        for i, s in enumerate(seqs):
            l = int(batch.seq_lens[s])
            k, v = data[s]
            slot = sub["bt"][i, (l - 1) // cfg.page_size] * cfg.page_size + (l - 1) % cfg.page_size
            oracle.kv_write_fp8(k[l - 1:l], v[l - 1:l], np.array([slot], np.int64),
                                cfg.page_size, sub["P"], synth.SCALE_PER_HEAD,
                                host_scales[0], host_scales[1], None, sub["kc"], sub["vc"])
        tags = np.zeros(sub["P"], np.uint32)
        ver = oracle.validate_page_tags(tags, sub["bt"], np.zeros(sub["bt"].shape, np.uint32),
                                        sub["lens"], cfg.page_size)
        oracle.paged_decode_attn(
            sub["q"], sub["kc"], sub["vc"], host_scales[0], host_scales[1], sub["bt"],
            sub["lens"], num_kv_heads=cfg.num_kv_heads, head_dim_v=cfg.head_dim_v,
            page_size=cfg.page_size, num_pages=sub["P"], kv_dtype=1, scale_mode=1,
            v_in_k=False, sm_scale=cfg.sm_scale, verdict=ver, num_threads=nthreads)
        return time.perf_counter() - t0

    seqs = list(range(8))
    sub = oracle_subset(batch, data, seqs, synth.KV_FP8, host_scales)
    t1 = run(seqs, sub)
    reps = int(max(1, min(100, round(target_s / max(t1, 1e-3)))))
    t = sum(run(seqs, sub) for _ in range(reps))
    n = len(seqs) * reps
    kvb = n * int(batch.seq_lens[0]) * cfg.num_kv_heads * (cfg.head_dim_qk + cfg.head_dim_v)
    from oracle.pool import OraclePagePool
    pool_rate = pool_cycles(OraclePagePool(32768, initial_order=np.random.default_rng(1)
                                           .permutation(32768)), 0.3)
    return {"value": kvb / t / 1e9, "unit": "GB/s", "cores": nthreads, "kind": "oracle",
            "seq_steps_per_s": n / t, "page_pool_pages_per_s": pool_rate,
            "int4_gemv": int4_oracle_rate(np, synth),
            "sample": f"{len(seqs)} whole sequences of the 64 x 8192 workload (all 64 query "
                      f"heads), {reps} steps: kv write of the newest token, tag check, fp64 "
                      f"attention; {t:.1f} s"}


def gen_data(batch, synth):
    return synth.map_seqs(lambda s: batch.kv(s), list(range(batch.B)),
                          min(16, os.cpu_count() or 1))


def latent_leg(args, torch, synth, pda, workload):
    """The latent workload (64 sequences of U[1024, 32768] tokens, 128 query
    heads, one 576-dim kv head, per-token scales) on the matrix-core path:
    the attention call timed like the metric's (median of interleaved
    passes of exactly K calls), rated against the dense bf16/f16 matrix
    peak. After the shared warm-up the leg makes LATENT_SETTLE_CALLS more
    untimed calls: under a kernel trace the partial kernel's time rises from
    ~320 to ~400 us a few calls after the memory-bound legs and settles at
    285-300 us after about 100 calls (the matrix-heavy kernel follows the
    chip's clock state; memory-bound kernels move 1-2 %), and the passes
    are meant to time the settled state a serving loop runs in."""
    batch = synth.make_batch(4)
    log("latent workload: generating inputs and cache")
    db = workload.build(batch, pda.KV_FP8_E4M3, data=gen_data(batch, synth))
    db.alloc_workspace()
    for _ in range(args.warmup):
        db.step()
    for _ in range(LATENT_SETTLE_CALLS):
        db.attend()
    torch.cuda.synchronize()
    t = interleaved_passes({"attn": lambda: db.attend()}, args.steps, args.passes, torch)
    attn_ms = median(t["attn"])
    flops = workload.attention_flops(batch)
    kv = workload.kv_bytes(batch, pda.KV_FP8_E4M3)
    tf = flops / (attn_ms * 1e-3) / 1e12
    log(f"latent attention call: {attn_ms:.4f} ms, {tf:.0f} TFLOP/s")
    out = {"workload": batch.cfg.name, "tokens": int(batch.seq_lens.sum()),
           "attn_ms": attn_ms, "attn_ms_passes": t["attn"],
           "untimed_calls_before_passes": args.warmup + LATENT_SETTLE_CALLS,
           "roofline": {"kernel": "paged_decode_attn latent (partial + combine)",
                        "bound": "mfma", "achieved": tf, "peak": MFMA_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": tf / MFMA_PEAK_TFLOPS,
                        "hbm_frac": kv / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS,
                        "algorithmic_flops_per_launch": flops, "traffic": None}}
    del db
    torch.cuda.empty_cache()
    return out


def full_pool_leg(args, torch, synth, pda, workload, overlap):
    """The full-pool workload (256 lognormal sequences, churned pool, one
    injected tag mismatch per 10,000 pages, 256 new tokens per step): whole
    steps with the tag check and with the no-op tracker, interleaved
    passes; the check's share of the step, and the attention call alone."""
    batch = synth.make_batch(5)
    log("full-pool workload: generating inputs and cache")
    db = workload.build(batch, pda.KV_FP8_E4M3, data=gen_data(batch, synth))
    db.alloc_workspace()
    for _ in range(args.warmup):
        db.step(overlap=overlap)
    t = interleaved_passes({"on": lambda: db.step(overlap=overlap),
                            "off": lambda: db.step(use_verdict=False),
                            "two_launches": lambda: db.step(fused=False),
                            "attn": lambda: db.attend()}, args.steps, args.passes, torch)
    bd = breakdown(db, args.steps, torch)
    on, off, attn = median(t["on"]), median(t["off"]), median(t["attn"])
    kv = workload.kv_bytes(batch, pda.KV_FP8_E4M3)
    log(f"full pool: step {on:.4f} ms (no-op tracker {off:.4f}), attention {attn:.4f} ms")
    out = {"workload": batch.cfg.name, "tokens": int(batch.seq_lens.sum()),
           "step_ms": on, "step_ms_no_op_tracker": off, "attn_ms": attn,
           "tag_check_overhead_frac": median([a / b for a, b in zip(t["on"], t["off"])]) - 1.0,
           "step_ms_two_launches": median(t["two_launches"]),
           "tag_check_overhead_frac_two_launches":
               median([a / b for a, b in zip(t["two_launches"], t["off"])]) - 1.0,
           "write_check_ms": bd["write_check_ms"],
           "validate_ms": bd["validate_ms"], "validate_frac_of_step":
               bd["validate_ms"] / bd["step_ms_with_call_events"],
           "kv_write_ms": bd["kv_write_ms"],
           "seq_steps_per_s": batch.B / (on * 1e-3),
           "kv_GBps_step": kv / (on * 1e-3) / 1e9,
           "pct_hbm_peak_attn": 100.0 * kv / (attn * 1e-3) / 1e9 / HBM_PEAK_GBPS,
           "verdicts_nonzero": int((db.verdict.cpu().numpy() != 0).sum())}
    del db
    torch.cuda.empty_cache()
    return out


def sweep(args, torch, np, synth, pda, workload):
    """Kernel-level concurrency and capacity sweep: B sequences of 8192
    tokens (the 64 x 8192 workload's heads and outliers; automatic split-K,
    which keeps 512-token chunks from 32 sequences up and halves them below
    so that small batches still fill the chip) for B in 1, 8, 16, 32, 64,
    FP8 and BF16 caches, steps and attention calls timed in interleaved
    passes; plus cache bytes per token and tokens per GiB of pool."""
    rows = []
    for B in (1, 8, 16, 32, 64):
        batch = synth.make_batch(WORKLOAD_ID, lens=[8192] * B)
        data = gen_data(batch, synth)
        dbs = {}
        for name, dt in (("fp8", pda.KV_FP8_E4M3), ("bf16", pda.KV_BF16)):
            dbs[name] = workload.build(batch, dt, data=data)
            dbs[name].alloc_workspace(split_tokens=0)
            for _ in range(args.warmup):
                dbs[name].step()
        log(f"sweep B={B}")
        t = interleaved_passes({f"{n}_{w}": (lambda d=d, w=w: d.step() if w == "step"
                                             else d.attend())
                                for n, d in dbs.items() for w in ("step", "attn")},
                               args.steps, args.passes, torch)
        row = {"seqs": B}
        for name, dt in (("fp8", pda.KV_FP8_E4M3), ("bf16", pda.KV_BF16)):
            kv = workload.kv_bytes(batch, dt)
            step, attn = median(t[f"{name}_step"]), median(t[f"{name}_attn"])
            row[name] = {"split": "auto", "step_ms": step, "attn_ms": attn,
                         "seq_steps_per_s": B / (step * 1e-3),
                         "kv_GBps_attn": kv / (attn * 1e-3) / 1e9,
                         "pct_hbm_peak_attn": 100.0 * kv / (attn * 1e-3) / 1e9
                         / HBM_PEAK_GBPS}
        row["fp8_over_bf16_seq_steps"] = (row["fp8"]["seq_steps_per_s"]
                                          / row["bf16"]["seq_steps_per_s"])
        rows.append(row)
        del dbs, data
        torch.cuda.empty_cache()
    cfg = synth.CONFIGS[WORKLOAD_ID]
    per_tok = {"fp8": cfg.num_kv_heads * (cfg.head_dim_qk + cfg.head_dim_v),
               "bf16": 2 * cfg.num_kv_heads * (cfg.head_dim_qk + cfg.head_dim_v)}
    return {"metric": "kernel-level concurrency sweep, 8192-token contexts, FP8 vs BF16 KV",
            "unit": "seq-steps/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "passes": args.passes, "data": "synthetic", "rows": rows,
            "capacity": {"cache_bytes_per_token": per_tok,
                         "tokens_per_GiB": {k: (1 << 30) // v for k, v in per_tok.items()}}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--passes", type=int, default=7,
                    help="timed passes of exactly --steps steps per leg (median reported)")
    ap.add_argument("--schedule", choices=("serial", "overlap"), default=DEFAULT_SCHEDULE,
                    help="step schedule: every call on one stream, or the tag check on a "
                         "second stream beside the kv write (attention waits for both)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the latent, full-pool, transcode and INT4 legs")
    ap.add_argument("--sweep", action="store_true",
                    help="kernel-level concurrency sweep: 1..64 sequences of 8192 tokens, "
                         "FP8 and BF16; one JSON line")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy, whose HBM "
                         "counters calibrate FETCH_SIZE / WRITE_SIZE in a profiled run")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import decode_attention_fp8_write_amd as pda
    from synth import device as workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    pda.load()
    if args.copy_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        log("copy calibration: 1 GiB read + 1 GiB written by one copy kernel")
    if args.sweep:
        print(json.dumps(sweep(args, torch, np, synth, pda, workload)), flush=True)
        return
    overlap = args.schedule == "overlap"

    # page bookkeeping from the library's own pool and tag tracker
    # (pda_pool_*), checked against the harness pool it replaces
    batch = synth.make_batch(
        WORKLOAD_ID, pool_factory=lambda n, o: pda.PagePool(n, initial_order=o))
    ref_batch = synth.make_batch(WORKLOAD_ID)
    pool_same = bool(np.array_equal(batch.block_table, ref_batch.block_table)
                     and np.array_equal(batch.expected_tags, ref_batch.expected_tags)
                     and np.array_equal(batch.page_tags, ref_batch.page_tags))
    assert pool_same, "library page pool and harness pool disagree"
    del ref_batch
    cfg = batch.cfg
    B = batch.B
    log("generating inputs")
    data = gen_data(batch, synth)
    log("building FP8 and BF16 caches")
    fp8 = workload.build(batch, pda.KV_FP8_E4M3, data=data)
    fp8.alloc_workspace()
    bf = workload.build(batch, pda.KV_BF16, data=data)
    bf.alloc_workspace()
    for _ in range(args.warmup):
        fp8.step(overlap=overlap)
        bf.step(overlap=overlap)
    log(f"timing {args.passes} interleaved passes of {args.steps} steps ({args.schedule})")
    # the step with and without the check run next to each other in every
    # round, so that the check's share is taken pass by pass (drift between
    # legs further apart in a round was as large as the check itself)
    t = interleaved_passes({
        "fp8_step": lambda: fp8.step(overlap=overlap),
        "fp8_step_no_op_tracker": lambda: fp8.step(use_verdict=False),
        "fp8_step_two_launches": lambda: fp8.step(fused=False),
        "bf16_step": lambda: bf.step(overlap=overlap),
        "fp8_attn": lambda: fp8.attend(),
        "bf16_attn": lambda: bf.attend(),
        "fp8_step_other_schedule": lambda: fp8.step(overlap=not overlap),
        "bf16_step_other_schedule": lambda: bf.step(overlap=not overlap),
    }, args.steps, args.passes, torch)
    med = {k: median(v) for k, v in t.items()}
    for k, v in med.items():
        log(f"  {k}: {v:.4f} ms (passes {', '.join(f'{x:.4f}' for x in t[k])})")
    bd8 = breakdown(fp8, args.steps, torch)
    bd16 = breakdown(bf, args.steps, torch)
    kv8 = workload.kv_bytes(batch, pda.KV_FP8_E4M3)
    kv16 = workload.kv_bytes(batch, pda.KV_BF16)
    step8, step16 = med["fp8_step"], med["bf16_step"]
    attn8, attn16 = med["fp8_attn"], med["bf16_attn"]
    # algorithmic bytes of one attention call: KV, q, out, block-table entries
    q_bytes = B * cfg.num_q_heads * cfg.head_dim_qk * 2
    out_bytes = B * cfg.num_q_heads * cfg.head_dim_v * 4
    bt_bytes = int(np.sum(-(-batch.seq_lens // cfg.page_size))) * 4
    attn_bytes = kv8 + q_bytes + out_bytes + bt_bytes
    achieved = attn_bytes / (attn8 * 1e-3) / 1e9
    seq_steps = B / (step8 * 1e-3)
    seq_steps16 = B / (step16 * 1e-3)
    res_bf16 = {"step_ms": step16, "attn_ms": attn16, "seq_steps_per_s": seq_steps16,
                "kv_GBps_step": kv16 / (step16 * 1e-3) / 1e9,
                "kv_GBps_attn": kv16 / (attn16 * 1e-3) / 1e9,
                "step_ms_passes": t["bf16_step"], "attn_ms_passes": t["bf16_attn"],
                "step_ms_other_schedule": med["bf16_step_other_schedule"],
                "validate_ms": bd16["validate_ms"], "kv_write_ms": bd16["kv_write_ms"]}
    ceiling = read_ceiling(torch, pda)
    extra = {}
    if not args.no_extra:
        log("timing the BF16 -> FP8 page transcode of the whole pool")
        res_bf16["transcode"] = time_transcode(bf, fp8, args, torch, np, pda)
    del bf
    torch.cuda.empty_cache()
    if not args.no_extra:
        extra["latent_workload"] = latent_leg(args, torch, synth, pda, workload)
        extra["full_pool_workload"] = full_pool_leg(args, torch, synth, pda, workload, overlap)
        log("timing the INT4 weight-only GEMV")
        extra["int4_gemv"] = time_int4(torch, pda)

    line = {
        "metric": METRIC,
        "value": kv8 / (step8 * 1e-3) / 1e9,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": step8,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 KV, bf16/f16 dot2 operands, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "64 seqs x 8192 ctx, 64 q / 8 kv heads, d128, page 16, "
                               "FP8 e4m3 KV (per-head scales; K 6/128 channels x20), "
                               "split-K 512; step = kv write of 64 new tokens and tag "
                               "validation (one launch) + attention",
                   "global_batch": B, "seq_len": int(batch.seq_lens[0]),
                   "parallelism": "single GPU"},
        "timing": f"median of {args.passes} interleaved passes of exactly {args.steps} "
                  f"steps (FP8, BF16 and the other legs alternate) after {args.warmup} "
                  f"warm-up steps of each",
        "schedule": args.schedule,
        "pct_hbm_peak_step": 100.0 * kv8 / (step8 * 1e-3) / 1e9 / HBM_PEAK_GBPS,
        "seq_steps_per_s": seq_steps,
        "tokens_per_s": seq_steps,
        "step_ms_passes": t["fp8_step"],
        "step_ms_other_schedule": med["fp8_step_other_schedule"],
        "attn_ms": attn8,
        "attn_ms_passes": t["fp8_attn"],
        "validate_ms": bd8["validate_ms"],
        "kv_write_ms": bd8["kv_write_ms"],
        "validate_frac_of_step": bd8["validate_ms"] / bd8["step_ms_with_call_events"],
        "step_ms_with_call_events": bd8["step_ms_with_call_events"],
        "tag_check": {"step_ms_check_on": step8,
                      "step_ms_check_off": med["fp8_step_no_op_tracker"],
                      "overhead_frac": median([a / b for a, b in zip(
                          t["fp8_step"], t["fp8_step_no_op_tracker"])]) - 1.0,
                      "overhead_frac_of_medians": step8 / med["fp8_step_no_op_tracker"] - 1.0,
                      "step_ms_two_launches": med["fp8_step_two_launches"],
                      "overhead_frac_two_launches": median([a / b for a, b in zip(
                          t["fp8_step_two_launches"], t["fp8_step_no_op_tracker"])]) - 1.0,
                      "write_check_ms": bd8["write_check_ms"],
                      "tags_from": "libpda.so page pool (pda_pool_*), identical to the "
                                   "harness pool's bookkeeping"},
        "page_pool": time_page_pool(pda, np),
        "hbm_read_ceiling": ceiling,
        "kv_GBps_attn": kv8 / (attn8 * 1e-3) / 1e9,
        "fp8_over_bf16_seq_steps": seq_steps / seq_steps16,
        "fp8_over_bf16_attn": attn16 / attn8,
        "bf16": res_bf16,
        "roofline": {"kernel": "paged_decode_attn (attn_partial + attn_combine)",
                     "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS,
                     "algorithmic_bytes_per_launch": attn_bytes,
                     "frac_of_measured_read_ceiling":
                         achieved / max(ceiling.values()),
                     "traffic": measured_traffic()},
    }
    line.update(extra)
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        line["cpu_baseline"] = cpu_baseline(batch, data, fp8.host_scales)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
