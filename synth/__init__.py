"""Seeded synthetic inputs for the FP8 paged decode-attention path.

This module generates INPUTS only and is shared by the GPU tests, the
benchmark and the oracle tests: BF16 sampling, sequence lengths, query
vectors, per-head scales (amax/448 of the data a run will write), the
physical page pool with its per-page tags (the host-side bookkeeping of the
integrity check), block tables, expected-tag records, mismatch injection and
poison values. None of the path's arithmetic — quantisation, validation,
attention — lives here.

Workloads (all head counts, dims and page sizes as named):
  1  tiny step: 4 sequences of lengths {17, 64, 100, 255}, 8 query / 2 kv
     heads, dim 128, pages of 16, a pool of 64 pages handed out by a seeded
     permutation, one injected tag mismatch, unused pages poisoned.
  2  32 x 8192 tokens, 64 / 8 heads, dim 128, pages of 16; BF16 and FP8
     caches; one new token written per sequence per step.
  3  64 x 8192 tokens, FP8, 64 / 8 heads, dim 128, pages of 16; K has 6 of
     128 channels per kv head scaled by 20; split-K chunks of 512 tokens.
  4  latent: one kv head of 576 dims (V = its first 512), 128 query heads,
     64 sequences of lengths uniform in [1024, 32768], pages of 64, FP8 with
     one scale per token.
  5  full pool: 256 sequences, lognormal lengths (median 4096, sigma 0.656,
     cap 65536), 64 / 8 heads, dim 128, pages of 16, pool fragmented by
     seeded allocate/free churn, 32-bit page tags, one mismatch injected per
     10,000 pages in use, one new token per sequence per step.

Seeds: numpy SeedSequence(1000 + workload id) with one spawn key per stream
(queries, lengths, pool, outlier channels, injection, and one key per
sequence for its K/V), so any sequence's data can be regenerated alone.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# stream ids (spawn keys)
_Q, _LENS, _POOL, _OUTLIER, _INJECT, _KV = 0, 1, 2, 3, 4, 6

KV_BF16, KV_FP8 = 0, 1
SCALE_NONE, SCALE_PER_HEAD, SCALE_PER_TOKEN = 0, 1, 2

FP8_POISON = 0x7F      # e4m3 NaN code
BF16_POISON = 0x7FC0   # bf16 quiet NaN


def rng_for(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(
        np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def bf16_from_f32(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 bit patterns, nearest-even; NaN -> quiet NaN."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    r = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))))
         >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return r


def bf16_to_f32(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    num_seqs: int
    num_q_heads: int
    num_kv_heads: int
    head_dim_qk: int
    head_dim_v: int
    page_size: int
    kv_dtypes: tuple
    scale_mode: int          # for the FP8 cache
    v_in_k: bool
    split_tokens: int        # 0 = automatic
    outlier_channels: int    # per kv head, K only
    outlier_mult: float
    new_tokens_per_step: int
    max_len: int             # longest possible sequence of the workload

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def seed(self) -> int:
        return 1000 + self.cid

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim_qk)

    @property
    def max_blocks(self) -> int:
        return -(-self.max_len // self.page_size)


CONFIGS = {
    1: Config(1, "tiny: 4 seqs {17,64,100,255}, 8/2 heads, d128, S16, 64 pages",
              4, 8, 2, 128, 128, 16, (KV_FP8, KV_BF16), SCALE_PER_HEAD, False,
              0, 0, 1.0, 0, 255),
    2: Config(2, "32 x 8192 ctx, 64/8 heads, d128, S16, BF16 and FP8 KV",
              32, 64, 8, 128, 128, 16, (KV_BF16, KV_FP8), SCALE_PER_HEAD,
              False, 0, 0, 1.0, 32, 8192),
    3: Config(3, "64 x 8192 ctx, FP8 KV, 64/8 heads, d128, S16, K outliers, "
                 "split 512", 64, 64, 8, 128, 128, 16, (KV_FP8, KV_BF16),
              SCALE_PER_HEAD, False, 512, 6, 20.0, 0, 8192),
    4: Config(4, "latent: 1 kv head d576 (V = first 512), 128 q heads, 64 "
                 "seqs U[1024,32768], S64, FP8 per-token scale",
              64, 128, 1, 576, 512, 64, (KV_FP8,), SCALE_PER_TOKEN, True, 0,
              0, 1.0, 0, 32768),
    5: Config(5, "full pool: 256 seqs lognormal (median 4k, cap 64k), 64/8 "
                 "heads, d128, S16, churned pool, 1 mismatch / 10k pages",
              256, 64, 8, 128, 128, 16, (KV_FP8,), SCALE_PER_HEAD, False, 0,
              0, 1.0, 256, 65536),
}


def config_lengths(cfg: Config) -> np.ndarray:
    rng = rng_for(cfg.seed, _LENS)
    if cfg.cid == 1:
        lens = [17, 64, 100, 255]
    elif cfg.cid in (2, 3):
        lens = [8192] * cfg.num_seqs
    elif cfg.cid == 4:
        lens = rng.integers(1024, 32768, size=cfg.num_seqs, endpoint=True)
    elif cfg.cid == 5:
        x = rng.lognormal(mean=math.log(4096.0), sigma=0.656, size=cfg.num_seqs)
        lens = np.clip(np.rint(x), 1, 65536)
    else:
        raise ValueError(cfg.cid)
    return np.asarray(lens, dtype=np.int32)


class PagePool:
    """Physical page pool with a global 32-bit allocation counter.

    Every hand-out of a page stamps it with the next counter value, so a page
    that is freed and handed out again carries a new tag, and tags are unique
    among pages in use (until the counter wraps). Free pages are kept on a
    stack: the most recently freed page is handed out first."""

    def __init__(self, num_pages: int, rng: Optional[np.random.Generator] = None,
                 tag_start: int = 0, order=None):
        self.num_pages = num_pages
        self.tags = np.zeros(num_pages, dtype=np.uint32)
        self.counter = int(tag_start) & 0xFFFFFFFF
        # initial free stack in a seeded order (or the given order of the
        # first hand-outs); pop() takes from the end
        if order is None:
            order = rng.permutation(num_pages)
        self._free = [int(p) for p in np.asarray(order)[::-1]]

    @property
    def num_free(self) -> int:
        return len(self._free)

    def alloc(self, n: int):
        if n > len(self._free):
            raise MemoryError("page pool exhausted")
        pages = np.empty(n, dtype=np.int32)
        tags = np.empty(n, dtype=np.uint32)
        for i in range(n):
            p = self._free.pop()
            self.counter = (self.counter + 1) & 0xFFFFFFFF
            self.tags[p] = self.counter
            pages[i] = p
            tags[i] = self.counter
        return pages, tags

    def free(self, pages) -> None:
        for p in pages:
            self._free.append(int(p))

    def free_pages(self) -> np.ndarray:
        return np.asarray(self._free, dtype=np.int32)


@dataclass
class Batch:
    cfg: Config
    seq_lens: np.ndarray        # int32 [B]
    num_pages: int
    block_table: np.ndarray     # int32 [B, max_blocks], -1 padding
    expected_tags: np.ndarray   # uint32 [B, max_blocks], 0 padding
    page_tags: np.ndarray       # uint32 [P] (after injection)
    injected: list              # [(seq, block)] whose page tag was bumped
    q: np.ndarray               # uint16 bf16 [B, Hq, Dk]
    max_blocks: int
    _scales: Optional[tuple] = field(default=None, repr=False)

    @property
    def B(self) -> int:
        return int(self.seq_lens.shape[0])

    def used_pages(self) -> np.ndarray:
        used = []
        for s in range(self.B):
            n = -(-int(self.seq_lens[s]) // self.cfg.page_size)
            used.append(self.block_table[s, :n])
        return np.concatenate(used) if used else np.zeros(0, np.int32)

    def slots(self, s: int, positions) -> np.ndarray:
        S = self.cfg.page_size
        pos = np.asarray(positions, dtype=np.int64)
        return (self.block_table[s, pos // S].astype(np.int64) * S + pos % S)

    def kv(self, s: int):
        """bf16 bit patterns of sequence s for positions [0, len):
        K [len, Hkv, Dk] and V [len, Hkv, Dv] (V None for latent caches)."""
        return seq_kv(self.cfg, s, int(self.seq_lens[s]))

    def scales(self, threads: Optional[int] = None):
        """Per-kv-head fp32 scales amax/448 over every K (resp. V) value the
        batch writes; amax == 0 gives 1.0. None for per-token scaling."""
        if self.cfg.scale_mode != SCALE_PER_HEAD:
            return None, None
        if self._scales is None:
            hkv = self.cfg.num_kv_heads

            def one(s):
                k, v = self.kv(s)
                ka = np.abs(bf16_to_f32(k)).reshape(-1, hkv, k.shape[-1]).max(axis=(0, 2))
                va = np.abs(bf16_to_f32(v)).reshape(-1, hkv, v.shape[-1]).max(axis=(0, 2))
                return ka, va

            res = map_seqs(one, [s for s in range(self.B) if self.seq_lens[s] > 0],
                           threads)
            kam = np.zeros(hkv, np.float32)
            vam = np.zeros(hkv, np.float32)
            for ka, va in res:
                kam = np.maximum(kam, ka)
                vam = np.maximum(vam, va)
            ks = np.where(kam > 0, kam / np.float32(448.0), np.float32(1.0))
            vs = np.where(vam > 0, vam / np.float32(448.0), np.float32(1.0))
            self._scales = (ks.astype(np.float32), vs.astype(np.float32))
        return self._scales


def map_seqs(fn, seqs, threads: Optional[int] = None):
    threads = threads or min(16, os.cpu_count() or 1)
    if threads <= 1 or len(seqs) <= 1:
        return [fn(s) for s in seqs]
    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(fn, seqs))


def outlier_channels(cfg: Config) -> np.ndarray:
    """[Hkv, n] K channel indices scaled by cfg.outlier_mult."""
    if cfg.outlier_channels == 0:
        return np.zeros((cfg.num_kv_heads, 0), dtype=np.int64)
    rng = rng_for(cfg.seed, _OUTLIER)
    return np.stack([np.sort(rng.choice(cfg.head_dim_qk, cfg.outlier_channels,
                                        replace=False))
                     for _ in range(cfg.num_kv_heads)])


def seq_kv(cfg: Config, s: int, length: int):
    rng = rng_for(cfg.seed, _KV, s)
    hkv = cfg.num_kv_heads
    k = rng.standard_normal((length, hkv, cfg.head_dim_qk), dtype=np.float32)
    if cfg.outlier_channels:
        ch = outlier_channels(cfg)
        for h in range(hkv):
            k[:, h, ch[h]] *= np.float32(cfg.outlier_mult)
    kb = bf16_from_f32(k)
    if cfg.v_in_k:
        return kb, None
    v = rng.standard_normal((length, hkv, cfg.head_dim_v), dtype=np.float32)
    return kb, bf16_from_f32(v)


def make_q(cfg: Config, num_seqs: int) -> np.ndarray:
    rng = rng_for(cfg.seed, _Q)
    q = rng.standard_normal((num_seqs, cfg.num_q_heads, cfg.head_dim_qk),
                            dtype=np.float32)
    return bf16_from_f32(q)


def _tags_of(pool) -> np.ndarray:
    t = pool.tags
    return np.asarray(t() if callable(t) else t, dtype=np.uint32).copy()


def make_batch(cid: int, lens=None, num_pages: Optional[int] = None,
               inject: Optional[int] = None, pool_factor: float = 1.2,
               churn_rounds: int = 6, pool_factory=None) -> Batch:
    """Build the page bookkeeping and queries of a workload.

    lens overrides the workload's lengths (for scaled-down parity runs).
    inject overrides the number of injected tag mismatches (default: 1 for
    workload 1, floor(pages in use / 10000) for workload 5, else 0).
    pool_factory(num_pages, order) -> pool replaces this module's PagePool
    by another pool with the same interface (alloc(n) -> (pages, tags),
    free(pages), num_free, num_pages, tags) whose first hand-outs follow
    `order`, e.g. the library's own page pool; the seeded sequence of pool
    operations is the same."""
    cfg = CONFIGS[cid]
    seq_lens = config_lengths(cfg) if lens is None else np.asarray(lens, np.int32)
    B = int(seq_lens.shape[0])
    S = cfg.page_size
    npages = [-(-int(l) // S) for l in seq_lens]
    used = int(sum(npages))
    max_blocks = max(cfg.max_blocks, max(npages) if npages else 1)
    prng = rng_for(cfg.seed, _POOL)
    if cid == 5:
        P = num_pages or int(math.ceil(pool_factor * used / 64.0)) * 64
    else:
        P = num_pages or (64 if cid == 1 else max(used, 1))
    order = prng.permutation(P)
    pool = (pool_factory or (lambda n, o: PagePool(n, order=o)))(P, order)
    if cid == 5:
        _churn(pool, cfg, prng, churn_rounds)
    block_table = np.full((B, max_blocks), -1, dtype=np.int32)
    expected = np.zeros((B, max_blocks), dtype=np.uint32)
    for s in range(B):
        pages, tags = pool.alloc(npages[s])
        block_table[s, :npages[s]] = pages
        expected[s, :npages[s]] = tags
    page_tags = _tags_of(pool)
    if inject is None:
        inject = 1 if cid == 1 else (used // 10000 if cid == 5 else 0)
    injected = []
    if inject:
        irng = rng_for(cfg.seed, _INJECT)
        flat = irng.choice(used, size=inject, replace=False)
        starts = np.cumsum([0] + npages)
        for f in sorted(int(x) for x in flat):
            s = int(np.searchsorted(starts, f, side="right") - 1)
            j = f - int(starts[s])
            page_tags[block_table[s, j]] += np.uint32(1)
            injected.append((s, j))
    q = make_q(cfg, B)
    return Batch(cfg, seq_lens, P, block_table, expected, page_tags, injected,
                 q, max_blocks)


def _churn(pool, cfg: Config, rng: np.random.Generator,
           rounds: int) -> None:
    """Seeded rounds of handing out pages to short-lived sequences and freeing
    a random half of them, then freeing the rest, so the free stack the live
    sequences draw from is scattered over the pool."""
    S = cfg.page_size
    live = []
    for _ in range(rounds):
        while True:
            n = -(-int(min(65536, max(1, rng.lognormal(math.log(4096.0), 0.656)))) // S)
            if n > pool.num_free - pool.num_pages // 4:
                break
            pages, _ = pool.alloc(n)
            live.append(pages)
        order = rng.permutation(len(live))
        keep = []
        for i, idx in enumerate(order):
            if i % 2 == 0:
                pool.free(live[idx])
            else:
                keep.append(live[idx])
        live = keep
    for idx in rng.permutation(len(live)):
        pool.free(live[idx])


def poison_value(kv_dtype: int) -> int:
    return FP8_POISON if kv_dtype == KV_FP8 else BF16_POISON
