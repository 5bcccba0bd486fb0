"""The oracle-side workload helpers the full-size GPU parity tests rely on:
a whole-pool oracle cache at the workload's own page ids gives the same
attention rows, bit for bit, as the compact per-sequence cache (attention
does not depend on where the pages sit), and leaves every page no sequence
owns at the poison value."""
import numpy as np

import oracle
import synth
from oracle.harness import (oracle_attn_full, oracle_attn_subset, oracle_full_cache,
                            oracle_subset)


def _check(cid, kv_dtype, lens=None):
    b = synth.make_batch(cid, lens=lens)
    data = [b.kv(s) for s in range(b.B)]
    scales = b.scales() if b.cfg.scale_mode == synth.SCALE_PER_HEAD else (None, None)
    if kv_dtype == synth.KV_BF16:
        scales = (None, None)
    kc, vc, ts = oracle_full_cache(b, data, kv_dtype, scales)
    verdict = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags,
                                        b.seq_lens, b.cfg.page_size)
    full = oracle_attn_full(b, kc, vc, ts, kv_dtype, scales, verdict)
    sub = oracle_subset(b, data, list(range(b.B)), kv_dtype, scales)
    compact = oracle_attn_subset(b, sub, kv_dtype, scales, verdict=verdict)
    assert np.array_equal(full, compact)
    # pages nobody owns keep the poison
    used = set(int(p) for p in b.used_pages())
    free = [p for p in range(b.num_pages) if p not in used]
    pe = b.cfg.num_kv_heads * b.cfg.page_size * b.cfg.head_dim_qk
    poison = synth.poison_value(kv_dtype)
    for p in free:
        assert np.all(kc[p * pe:(p + 1) * pe] == poison)
    return verdict


def test_full_cache_matches_compact_cache_tiny_fp8():
    verdict = _check(1, synth.KV_FP8)
    assert (verdict != 0).sum() == 1


def test_full_cache_matches_compact_cache_tiny_bf16():
    _check(1, synth.KV_BF16)


def test_full_cache_matches_compact_cache_latent():
    _check(4, synth.KV_FP8, lens=[70, 1, 129])
