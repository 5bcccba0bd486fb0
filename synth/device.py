"""Device-resident synthetic workloads for the benchmark, the smoke check
and the GPU tests (harness side of the library's boundary).

Builds one decode step's inputs on the GPU from the seeded generator in
``synth`` (input generation only) through the library's own calls: the
context of every sequence is written into the paged cache with
kv_write_fp8 / kv_write_bf16, exactly as a serving step would. Nothing here
computes any step of the path itself. Importing this module loads the
library's Python binding; ``synth`` itself does not.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

import synth
from decode_attention_fp8_write_amd import (
    KV_BF16, KV_FP8_E4M3, SCALE_NONE, SCALE_PER_HEAD, SCALE_PER_TOKEN, kv_write_bf16,
    kv_write_check, kv_write_fp8, make_shape, paged_decode_attn, paged_decode_attn_workspace_bytes,
    validate_page_tags)


def _u16(torch, a: np.ndarray):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16))


@dataclass
class DeviceBatch:
    batch: synth.Batch
    kv_dtype: int
    q: object
    k_cache: object
    v_cache: object
    k_scale: object          # per head [Hkv] or token scales [P*S] (latent)
    v_scale: object
    block_table: object
    expected_tags: object
    page_tags: object
    seq_lens: object
    verdict: object
    out: object
    step_k: object = None    # bf16 [B, Hkv, Dk]: the token at position len-1
    step_v: object = None
    step_slots: object = None
    host_scales: tuple = field(default=(None, None))
    workspace: object = None
    shape: object = None
    _side: object = None
    _fork: object = None
    _join: object = None

    @property
    def cfg(self):
        return self.batch.cfg

    @property
    def max_seq_len(self) -> int:
        return int(self.batch.seq_lens.max()) if self.batch.B else 0

    def make_shape(self, split_tokens: Optional[int] = None):
        cfg = self.cfg
        fp8 = self.kv_dtype == KV_FP8_E4M3
        mode = (SCALE_PER_TOKEN if cfg.v_in_k else SCALE_PER_HEAD) if fp8 else SCALE_NONE
        return make_shape(
            num_seqs=self.batch.B, num_q_heads=cfg.num_q_heads, num_kv_heads=cfg.num_kv_heads,
            head_dim_qk=cfg.head_dim_qk, head_dim_v=cfg.head_dim_v, page_size=cfg.page_size,
            num_pages=self.batch.num_pages, max_blocks_per_seq=self.batch.max_blocks,
            kv_dtype=self.kv_dtype, scale_mode=mode, v_in_k=cfg.v_in_k,
            split_tokens=cfg.split_tokens if split_tokens is None else split_tokens,
            sm_scale=cfg.sm_scale)

    def alloc_workspace(self, split_tokens: Optional[int] = None, nbytes: Optional[int] = None):
        import torch
        self.shape = self.make_shape(split_tokens)
        if nbytes is None:
            nbytes = paged_decode_attn_workspace_bytes(self.shape, self.max_seq_len)
        self.workspace = torch.empty(int(nbytes), dtype=torch.uint8, device=self.q.device)
        return self.workspace

    # --- the three steps of one decode step --------------------------------
    def write_step(self, stream=None):
        """Write each sequence's newest token (position len-1) again."""
        if self.step_k is None:
            return
        S, P = self.cfg.page_size, self.batch.num_pages
        if self.kv_dtype == KV_FP8_E4M3:
            if self.cfg.v_in_k:
                kv_write_fp8(self.step_k, None, self.step_slots, self.k_cache, None,
                             page_size=S, num_pages=P, scale_mode=SCALE_PER_TOKEN,
                             token_scale=self.k_scale, stream=stream)
            else:
                kv_write_fp8(self.step_k, self.step_v, self.step_slots, self.k_cache,
                             self.v_cache, page_size=S, num_pages=P,
                             scale_mode=SCALE_PER_HEAD, k_scale=self.k_scale,
                             v_scale=self.v_scale, stream=stream)
        else:
            kv_write_bf16(self.step_k, self.step_v, self.step_slots, self.k_cache,
                          self.v_cache, page_size=S, num_pages=P, stream=stream)

    def write_check(self, stream=None):
        """write_step and validate in one launch (kv_write_check)."""
        S, P = self.cfg.page_size, self.batch.num_pages
        if self.step_k is None:
            self.validate(stream)
            return
        fp8 = self.kv_dtype == KV_FP8_E4M3
        if fp8 and self.cfg.v_in_k:
            kw = dict(scale_mode=SCALE_PER_TOKEN, token_scale=self.k_scale)
        elif fp8:
            kw = dict(scale_mode=SCALE_PER_HEAD, k_scale=self.k_scale, v_scale=self.v_scale)
        else:
            kw = dict(scale_mode=SCALE_NONE)
        kv_write_check(self.step_k, None if self.cfg.v_in_k else self.step_v, self.step_slots,
                       self.k_cache, None if self.cfg.v_in_k else self.v_cache,
                       self.page_tags, self.block_table, self.expected_tags, self.seq_lens,
                       self.verdict, page_size=S, num_pages=P, kv_dtype=self.kv_dtype,
                       stream=stream, **kw)

    def validate(self, stream=None):
        validate_page_tags(self.page_tags, self.block_table, self.expected_tags,
                           self.seq_lens, self.verdict, page_size=self.cfg.page_size,
                           stream=stream)

    def attend(self, use_verdict: bool = True, stream=None):
        if self.workspace is None:
            self.alloc_workspace()
        ks = self.k_scale if self.kv_dtype == KV_FP8_E4M3 else None
        vs = (self.v_scale if (self.kv_dtype == KV_FP8_E4M3 and not self.cfg.v_in_k)
              else None)
        paged_decode_attn(self.shape, self.q, self.k_cache, self.v_cache, ks, vs,
                          self.block_table, self.seq_lens, self.max_seq_len,
                          self.verdict if use_verdict else None, self.workspace, self.out,
                          stream=stream)

    def step(self, use_verdict: bool = True, stream=None, overlap: bool = False,
             fused: bool = True):
        """One decode step: kv write of the newest tokens, the tag check,
        attention. fused: the write and the check share one launch
        (kv_write_check); otherwise they are two launches in a row.
        overlap: the tag check runs on a second stream (default priority)
        beside the kv write, which it does not depend on; attention waits for
        both."""
        if not (overlap and use_verdict):
            if use_verdict and fused:
                self.write_check(stream)
            else:
                self.write_step(stream)
                if use_verdict:
                    self.validate(stream)
            self.attend(use_verdict, stream)
            return
        import torch
        main = torch.cuda.current_stream() if stream is None else stream
        if self._side is None:
            self._side = torch.cuda.Stream(device=self.q.device)
            self._fork = torch.cuda.Event()
            self._join = torch.cuda.Event()
        # the check rewrites the verdicts the previous step's attention read
        self._fork.record(main)
        self._side.wait_event(self._fork)
        self.validate(self._side)
        self._join.record(self._side)
        self.write_step(main)
        main.wait_event(self._join)
        self.attend(True, main)


def build(batch: synth.Batch, kv_dtype: int, *, device: str = "cuda", data=None,
          poison: bool = True, threads: Optional[int] = None) -> DeviceBatch:
    """Allocate caches for `batch`, poison them, and write every context
    token through the kv_write kernel. data: optional list of per-sequence
    (k, v) bf16 arrays already generated (else generated here)."""
    import torch
    cfg = batch.cfg
    B, P, S = batch.B, batch.num_pages, cfg.page_size
    hkv, dk, dv = cfg.num_kv_heads, cfg.head_dim_qk, cfg.head_dim_v
    fp8 = kv_dtype == KV_FP8_E4M3
    if data is None:
        data = synth.map_seqs(lambda s: batch.kv(s), list(range(B)), threads)
    cdt = torch.uint8 if fp8 else torch.int16
    fill = synth.poison_value(synth.KV_FP8 if fp8 else synth.KV_BF16)
    if not fp8 and fill >= 0x8000:
        fill -= 0x10000
    k_cache = torch.full((P * hkv * S * dk,), fill if poison else 0, dtype=cdt, device=device)
    v_cache = None
    if not cfg.v_in_k:
        v_cache = torch.full((P * hkv * S * dv,), fill if poison else 0, dtype=cdt, device=device)
    host_scales = (None, None)
    if fp8 and cfg.v_in_k:
        k_scale = torch.full((P * S,), float("nan"), dtype=torch.float32, device=device)
        v_scale = None
    elif fp8:
        hkam = np.zeros(hkv, np.float32)
        hvam = np.zeros(hkv, np.float32)
        for k, v in data:
            if len(k):
                hkam = np.maximum(hkam, np.abs(synth.bf16_to_f32(k)).max(axis=(0, 2)))
                hvam = np.maximum(hvam, np.abs(synth.bf16_to_f32(v)).max(axis=(0, 2)))
        ks = np.where(hkam > 0, hkam / np.float32(448), np.float32(1)).astype(np.float32)
        vs = np.where(hvam > 0, hvam / np.float32(448), np.float32(1)).astype(np.float32)
        host_scales = (ks, vs)
        k_scale = torch.from_numpy(ks).to(device)
        v_scale = torch.from_numpy(vs).to(device)
    else:
        k_scale = v_scale = None
    db = DeviceBatch(
        batch=batch, kv_dtype=kv_dtype,
        q=_u16(torch, batch.q).to(device),
        k_cache=k_cache, v_cache=v_cache, k_scale=k_scale, v_scale=v_scale,
        block_table=torch.from_numpy(batch.block_table).to(device),
        expected_tags=torch.from_numpy(batch.expected_tags.view(np.int32)).to(device),
        page_tags=torch.from_numpy(batch.page_tags.view(np.int32)).to(device),
        seq_lens=torch.from_numpy(batch.seq_lens).to(device),
        verdict=torch.zeros(B, dtype=torch.int32, device=device),
        out=torch.empty((B, cfg.num_q_heads, dv), dtype=torch.float32, device=device),
        host_scales=host_scales)
    # write the context, a few sequences per launch
    pending = []
    ntok = 0
    for s in range(B):
        l = int(batch.seq_lens[s])
        if l == 0:
            continue
        pending.append(s)
        ntok += l
        if ntok >= 1 << 18 or s == B - 1:
            _write_seqs(db, data, pending)
            pending, ntok = [], 0
    if pending:
        _write_seqs(db, data, pending)
    # the per-step token: position len-1 of every non-empty sequence
    steps = [s for s in range(B) if batch.seq_lens[s] > 0]
    if steps:
        ks_ = np.stack([data[s][0][int(batch.seq_lens[s]) - 1] for s in steps])
        db.step_k = _u16(torch, ks_).to(device)
        if not cfg.v_in_k:
            vs_ = np.stack([data[s][1][int(batch.seq_lens[s]) - 1] for s in steps])
            db.step_v = _u16(torch, vs_).to(device)
        sl = np.array([batch.slots(s, [int(batch.seq_lens[s]) - 1])[0] for s in steps],
                      np.int64)
        db.step_slots = torch.from_numpy(sl).to(device)
    torch.cuda.synchronize()
    return db


def _write_seqs(db: DeviceBatch, data, seqs):
    import torch
    batch = db.batch
    device = db.q.device
    k = np.concatenate([data[s][0] for s in seqs])
    slots = np.concatenate([batch.slots(s, np.arange(int(batch.seq_lens[s]))) for s in seqs])
    kt = _u16(torch, k).to(device)
    st = torch.from_numpy(slots.astype(np.int64)).to(device)
    S, P = db.cfg.page_size, batch.num_pages
    if db.cfg.v_in_k:
        vt = None
    else:
        vt = _u16(torch, np.concatenate([data[s][1] for s in seqs])).to(device)
    if db.kv_dtype == KV_FP8_E4M3:
        if db.cfg.v_in_k:
            kv_write_fp8(kt, None, st, db.k_cache, None, page_size=S, num_pages=P,
                         scale_mode=SCALE_PER_TOKEN, token_scale=db.k_scale)
        else:
            kv_write_fp8(kt, vt, st, db.k_cache, db.v_cache, page_size=S, num_pages=P,
                         scale_mode=SCALE_PER_HEAD, k_scale=db.k_scale, v_scale=db.v_scale)
    else:
        kv_write_bf16(kt, vt, st, db.k_cache, db.v_cache, page_size=S, num_pages=P)


def kv_bytes(batch: synth.Batch, kv_dtype: int) -> int:
    """Algorithmic KV bytes one attention call reads: every context token of
    every kv head, K and V (latent: the shared entry once) plus per-token
    scales."""
    cfg = batch.cfg
    tokens = int(np.sum(batch.seq_lens.astype(np.int64)))
    elem = 1 if kv_dtype == KV_FP8_E4M3 else 2
    if cfg.v_in_k:
        return tokens * (cfg.head_dim_qk * elem + (4 if kv_dtype == KV_FP8_E4M3 else 0))
    return tokens * cfg.num_kv_heads * (cfg.head_dim_qk + cfg.head_dim_v) * elem


def attention_flops(batch: synth.Batch) -> int:
    cfg = batch.cfg
    tokens = int(np.sum(batch.seq_lens.astype(np.int64)))
    return 2 * cfg.num_q_heads * (cfg.head_dim_qk + cfg.head_dim_v) * tokens

