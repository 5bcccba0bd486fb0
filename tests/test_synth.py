"""CPU tests of the seeded input generator: BF16 rounding, workload shapes,
and the page pool's tag semantics (every page carries a tag that changes when
the page is handed out again — remio.ai, section "Sicherheit gemeinsamer
KV-Caches wird zum Produktionsthema"; manulx.blog, section "Bảo vệ bộ nhớ đệm
dùng chung")."""
import os

import numpy as np
import pytest
import torch

import synth


def test_bf16_rne_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        (rng.standard_normal(1000) * 1e-38).astype(np.float32),
        np.array([0.0, -0.0, np.inf, -np.inf, 65504.0], np.float32),
        # exact ties between two bf16 values
        (np.arange(1000, dtype=np.uint32) << 16 | 0x8000).view(np.float32),
    ])
    ours = synth.bf16_from_f32(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert synth.bf16_from_f32(np.array([np.nan], np.float32))[0] & 0x7FC0 == 0x7FC0


def test_bf16_to_f32_round_trip():
    b = np.arange(65536, dtype=np.uint16)
    f = synth.bf16_to_f32(b)
    fin = np.isfinite(f)
    assert np.array_equal(synth.bf16_from_f32(f[fin]), b[fin])


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_workload_shapes(cid):
    b = synth.make_batch(cid)
    cfg = b.cfg
    S = cfg.page_size
    assert b.q.shape == (cfg.num_seqs, cfg.num_q_heads, cfg.head_dim_qk)
    assert b.block_table.shape == (cfg.num_seqs, b.max_blocks)
    used = b.used_pages()
    assert len(np.unique(used)) == len(used)            # no page shared
    assert used.min() >= 0 and used.max() < b.num_pages
    assert len(used) == sum(-(-int(l) // S) for l in b.seq_lens)
    if cid == 1:
        assert list(b.seq_lens) == [17, 64, 100, 255] and b.num_pages == 64
        assert len(used) == 29
    if cid in (2, 3):
        assert np.all(b.seq_lens == 8192) and b.num_pages == len(used)
    if cid == 4:
        assert b.seq_lens.min() >= 1024 and b.seq_lens.max() <= 32768
    if cid == 5:
        assert b.seq_lens.max() <= 65536 and b.seq_lens.min() >= 1
        assert 1.0e6 < b.seq_lens.sum() < 1.7e6
        assert b.num_pages >= 1.15 * len(used)
        assert len(b.injected) == len(used) // 10000


def test_deterministic():
    a = synth.make_batch(5)
    b = synth.make_batch(5)
    assert np.array_equal(a.block_table, b.block_table)
    assert np.array_equal(a.page_tags, b.page_tags)
    assert np.array_equal(a.q, b.q)
    k1, v1 = synth.seq_kv(a.cfg, 7, 100)
    k2, v2 = synth.seq_kv(a.cfg, 7, 100)
    assert np.array_equal(k1, k2) and np.array_equal(v1, v2)
    k3, _ = synth.seq_kv(a.cfg, 8, 100)
    assert not np.array_equal(k1, k3)


def test_pool_tags_change_on_reallocation():
    pool = synth.PagePool(8, np.random.default_rng(1))
    pages, tags = pool.alloc(8)
    old = dict(zip(pages.tolist(), tags.tolist()))
    pool.free(pages[:3])
    p2, t2 = pool.alloc(3)
    assert set(p2.tolist()) == set(pages[:3].tolist())
    for p, t in zip(p2.tolist(), t2.tolist()):
        assert t != old[p] and pool.tags[p] == t
    live = np.concatenate([pages[3:], p2])
    assert len(np.unique(pool.tags[live])) == 8       # unique among live pages
    with pytest.raises(MemoryError):
        pool.alloc(1)


def test_pool_counter_wraps_32_bit():
    pool = synth.PagePool(4, np.random.default_rng(2), tag_start=0xFFFFFFFE)
    _, tags = pool.alloc(3)
    assert list(tags) == [0xFFFFFFFF, 0, 1]


def test_workload5_pool_is_fragmented():
    b = synth.make_batch(5)
    S = b.cfg.page_size
    # most consecutive logical blocks of a sequence are not physically adjacent
    adj = 0
    tot = 0
    for s in range(b.B):
        n = -(-int(b.seq_lens[s]) // S)
        row = b.block_table[s, :n]
        adj += int(np.sum(np.diff(row) == 1))
        tot += max(n - 1, 0)
    assert adj < 0.2 * tot
    # expected tags match the current tags except at injected positions
    for s in range(b.B):
        n = -(-int(b.seq_lens[s]) // S)
        mism = np.nonzero(b.page_tags[b.block_table[s, :n]] != b.expected_tags[s, :n])[0]
        assert set(mism.tolist()) == {j for (ss, j) in b.injected if ss == s}


def test_outlier_channels_workload3():
    cfg = synth.CONFIGS[3]
    ch = synth.outlier_channels(cfg)
    assert ch.shape == (8, 6)
    k, v = synth.seq_kv(cfg, 0, 2000)
    kf = synth.bf16_to_f32(k)
    for h in range(8):
        std = kf[:, h, :].std(axis=0)
        big = set(np.nonzero(std > 5)[0].tolist())
        assert big == set(ch[h].tolist())
    assert abs(synth.bf16_to_f32(v).std() - 1.0) < 0.02


def test_scales_are_amax_over_written_data():
    b = synth.make_batch(1)
    ks, vs = b.scales()
    kam = np.zeros(2, np.float32)
    for s in range(b.B):
        k, v = b.kv(s)
        kam = np.maximum(kam, np.abs(synth.bf16_to_f32(k)).max(axis=(0, 2)))
    assert np.array_equal(ks, (kam / np.float32(448)).astype(np.float32))
    assert vs.shape == (2,) and np.all(vs > 0)


def test_pages_capacity_figures_match_half_size_cache():
    """The pages report the cache holding about 686k tokens in BF16 and 1.37M
    in FP8 e4m3 (tests/golden/pages_capacity.txt). Our per-token cache bytes:
    FP8 stores one byte per element where BF16 stores two, and per-head
    scales add nothing per token, so capacity at equal memory doubles; the
    pages' ratio must agree within their rounding."""
    path = os.path.join(os.path.dirname(__file__), "golden", "pages_capacity.txt")
    vals = {}
    with open(path, encoding="utf-8") as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    hkv, d = 8, 128
    bf16_per_tok = hkv * 2 * d * 2
    fp8_per_tok = hkv * 2 * d * 1
    ratio = bf16_per_tok / fp8_per_tok
    pages_ratio = vals["fp8_tokens"] / vals["bf16_tokens"]
    assert abs(pages_ratio - ratio) / ratio <= 2 * vals["rounding_rel"]
    # per-token scales (latent layout: 576 codes + one fp32) cost 4/576
    assert abs((576 + 4) / 576 - 1.0069) < 1e-4
