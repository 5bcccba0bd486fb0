"""paged_decode_attn_noalloc (the fixed-scratch variant for callers that
cannot allocate) against paged_decode_attn with a caller workspace, through
the C ABI: two calls in a row on one device, the second smaller, for the
vector-ALU path (64 x 8192 FP8 workload, then the tiny 4-sequence workload
with an aborted sequence) and for the latent matrix-core path (8 sequences,
then 2); and the scratch-size error for shapes that cannot fit."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_attn_close, log, threads

pytestmark = pytest.mark.gpu


def _device_batch(pda, b, kv_dtype=None):
    from synth import device as workload
    kv_dtype = pda.KV_FP8_E4M3 if kv_dtype is None else kv_dtype
    data = synth.map_seqs(lambda s: b.kv(s), list(range(b.B)), threads())
    db = workload.build(b, kv_dtype, data=data)
    db.alloc_workspace()
    db.validate()
    return db


def _both(pda, db):
    """Output of the workspace entry point and of the no-allocation one, in
    that order, on the same inputs and stream."""
    db.attend(use_verdict=True)
    torch.cuda.synchronize()
    want = db.out.clone()
    db.out.fill_(float("nan"))
    ks = db.k_scale if db.kv_dtype == pda.KV_FP8_E4M3 else None
    vs = db.v_scale if (db.kv_dtype == pda.KV_FP8_E4M3 and not db.cfg.v_in_k) else None
    pda.paged_decode_attn_noalloc(db.shape, db.q, db.k_cache, db.v_cache, ks, vs,
                                  db.block_table, db.seq_lens, db.max_seq_len, db.verdict,
                                  db.out)
    torch.cuda.synchronize()
    return want.cpu().numpy(), db.out.cpu().numpy()


def _check(want, got, what):
    # the same kernels on the same plan: the bits must agree (and so does
    # the attention bar of the oracle comparisons, which is checked too)
    assert_attn_close(got, want, what)
    assert np.array_equal(np.isnan(got), np.isnan(want)), what
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok]), f"{what}: not bit-identical"


def test_noalloc_vector_alu_two_calls(gpu):
    pda = gpu
    log("no-alloc: 64 x 8192 FP8 workload, then the tiny workload")
    b3 = synth.make_batch(3)
    db3 = _device_batch(pda, b3)
    assert db3.workspace.numel() <= pda.paged_decode_attn_noalloc_scratch_bytes()
    want, got = _both(pda, db3)
    _check(want, got, "64 x 8192 no-alloc")
    del db3
    torch.cuda.empty_cache()
    b1 = synth.make_batch(1)
    db1 = _device_batch(pda, b1)
    want, got = _both(pda, db1)
    verdict = db1.verdict.cpu().numpy()
    assert (verdict != 0).sum() == 1
    assert np.all(got[verdict != 0] == 0)
    _check(want, got, "tiny workload no-alloc after the large one")
    # and the BF16 cache of the tiny workload, a third call
    db1b = _device_batch(pda, b1, pda.KV_BF16)
    want, got = _both(pda, db1b)
    _check(want, got, "tiny BF16 no-alloc")


def test_noalloc_latent_two_calls(gpu):
    pda = gpu
    log("no-alloc: latent, 8 sequences then 2")
    for lens in ([1024, 3000, 64, 7777, 20000, 1, 4095, 12345], [65, 2049]):
        b = synth.make_batch(4, lens=lens)
        db = _device_batch(pda, b)
        want, got = _both(pda, db)
        _check(want, got, f"latent no-alloc lens {lens}")


def test_noalloc_rejects_shapes_beyond_the_scratch(gpu):
    pda = gpu
    lib = pda.load()
    fake = ctypes.c_void_p(256)
    big = pda.make_shape(num_seqs=16384, num_q_heads=64, num_kv_heads=8, head_dim_qk=128,
                         head_dim_v=128, page_size=16, num_pages=1 << 20,
                         max_blocks_per_seq=64, kv_dtype=pda.KV_FP8_E4M3,
                         scale_mode=pda.SCALE_PER_HEAD, split_tokens=0, sm_scale=0.088)
    # 16384 x 8 partials of 8 x 130 fp32 (545 MB) cannot fit 96 MiB
    st = lib.paged_decode_attn_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake,
                                       fake, 1024, None, fake, None)
    assert st == pda.PDA_ERR_SCRATCH
    lat = pda.make_shape(num_seqs=2048, num_q_heads=128, num_kv_heads=1, head_dim_qk=576,
                         head_dim_v=512, page_size=64, num_pages=1 << 16,
                         max_blocks_per_seq=512, kv_dtype=pda.KV_FP8_E4M3,
                         scale_mode=pda.SCALE_PER_TOKEN, v_in_k=True, split_tokens=0,
                         sm_scale=1.0 / 24)
    st = lib.paged_decode_attn_noalloc(ctypes.byref(lat), fake, fake, None, fake, None, fake,
                                       fake, 1024, None, fake, None)
    assert st == pda.PDA_ERR_SCRATCH
    assert "scratch" in pda.status_string(pda.PDA_ERR_SCRATCH)
