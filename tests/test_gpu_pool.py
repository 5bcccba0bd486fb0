"""The library's host page pool and tag tracker (pda_pool_*) driving a GPU
decode step. Pages of five requests come from the library pool; one request
then finishes, its pages go back to the pool and are handed to a new request,
which writes its own context into them. The finished request is left in the
batch with its old block table and expected tags, the reuse the pages' tag
check exists to catch (manulx.blog, "Công thức của Cloudflare để phục vụ Kimi
và GLM", section "Bảo vệ bộ nhớ đệm dùng chung"). The pool's tags are
uploaded as page_tags; validate_page_tags and paged_decode_attn run on the
GPU and are compared with the oracle (which replays the same two rounds of
writes into its own cache): the stale request is aborted at the first of its
pages that was handed out again, its rows are zero, every other row matches.
With the no-op tracker (tags off, NULL verdict) the same step reads the new
owner's data for the stale request, and still matches the oracle run without
a verdict."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_helpers import assert_attn_close, log

pytestmark = pytest.mark.gpu

S, P, HKV, HQ, D = 16, 64, 2, 8, 128
LENS = [17, 64, 100, 255, 40]      # requests 0..4
NEW_LEN = 90                       # request 5, on request 2's freed pages
STALE = 2


def _bookkeeping(pda, track):
    rng = np.random.default_rng(5)
    pool = pda.PagePool(P, initial_order=rng.permutation(P), tag_start=1000,
                        track_tags=track)
    maxb = 16
    bt = np.full((6, maxb), -1, np.int32)
    exp = np.zeros((6, maxb), np.uint32)
    for s, l in enumerate(LENS):
        n = -(-l // S)
        bt[s, :n], exp[s, :n] = pool.alloc(n)
    n2 = -(-LENS[STALE] // S)
    pool.free(bt[STALE, :n2])          # request 2 finishes
    n5 = -(-NEW_LEN // S)
    bt[5, :n5], exp[5, :n5] = pool.alloc(n5)
    assert set(bt[5, :n5].tolist()) <= set(bt[STALE, :n2].tolist())   # same pages again
    tags = pool.tags()
    pool.close()
    return bt, exp, tags


def _inputs():
    cfg = synth.CONFIGS[1]
    lens = LENS + [NEW_LEN]
    kv = [synth.seq_kv(cfg, s, l) for s, l in enumerate(lens)]
    q = synth.make_q(cfg, len(lens))
    kam = np.max([np.abs(synth.bf16_to_f32(k)).max(axis=(0, 2)) for k, _ in kv], axis=0)
    vam = np.max([np.abs(synth.bf16_to_f32(v)).max(axis=(0, 2)) for _, v in kv], axis=0)
    ks = (kam / np.float32(448)).astype(np.float32)
    vs = (vam / np.float32(448)).astype(np.float32)
    return cfg, np.array(lens, np.int32), kv, q, ks, vs


def _slots(bt, s, l):
    t = np.arange(l, dtype=np.int64)
    return bt[s, t // S].astype(np.int64) * S + t % S


@pytest.mark.parametrize("track", [True, False])
def test_library_pool_drives_the_step(gpu, track):
    pda = gpu
    log(f"library pool step, tag tracking {'on' if track else 'off (no-op tracker)'}")
    bt, exp, tags = _bookkeeping(pda, track)
    if not track:
        assert np.all(tags == 0)
    cfg, lens, kv, q, ks, vs = _inputs()
    dev = "cuda"
    kc = torch.full((P * HKV * S * D,), synth.FP8_POISON, dtype=torch.uint8, device=dev)
    vc = kc.clone()
    okc = np.full(P * HKV * S * D, synth.FP8_POISON, np.uint8)
    ovc = okc.copy()
    ks_t, vs_t = torch.from_numpy(ks).to(dev), torch.from_numpy(vs).to(dev)
    u16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    # first batch: requests 0..4; second batch: request 5 into request 2's old pages
    for seqs in ([0, 1, 2, 3, 4], [5]):
        k = np.concatenate([kv[s][0] for s in seqs])
        v = np.concatenate([kv[s][1] for s in seqs])
        sl = np.concatenate([_slots(bt, s, int(lens[s])) for s in seqs])
        pda.kv_write_fp8(u16(k), u16(v), torch.from_numpy(sl).to(dev), kc, vc, page_size=S,
                         num_pages=P, scale_mode=pda.SCALE_PER_HEAD, k_scale=ks_t, v_scale=vs_t)
        oracle.kv_write_fp8(k, v, sl, S, P, synth.SCALE_PER_HEAD, ks, vs, None, okc, ovc)
    bt_t = torch.from_numpy(bt).to(dev)
    lens_t = torch.from_numpy(lens).to(dev)
    verdict_t = torch.full((6,), -7, dtype=torch.int32, device=dev)
    out = torch.empty((6, HQ, D), dtype=torch.float32, device=dev)
    shape = pda.make_shape(num_seqs=6, num_q_heads=HQ, num_kv_heads=HKV, head_dim_qk=D,
                           head_dim_v=D, page_size=S, num_pages=P, max_blocks_per_seq=16,
                           kv_dtype=pda.KV_FP8_E4M3, scale_mode=pda.SCALE_PER_HEAD,
                           split_tokens=0, sm_scale=cfg.sm_scale)
    ws = torch.empty(pda.paged_decode_attn_workspace_bytes(shape, int(lens.max())),
                     dtype=torch.uint8, device=dev)
    if track:
        pda.validate_page_tags(torch.from_numpy(tags.view(np.int32)).to(dev), bt_t,
                               torch.from_numpy(exp.view(np.int32)).to(dev), lens_t, verdict_t,
                               page_size=S)
    pda.paged_decode_attn(shape, u16(q), kc, vc, ks_t, vs_t, bt_t, lens_t, int(lens.max()),
                          verdict_t if track else None, ws, out)
    torch.cuda.synchronize()
    assert np.array_equal(kc.cpu().numpy(), okc) and np.array_equal(vc.cpu().numpy(), ovc)
    want_verdict = None
    if track:
        want_verdict = oracle.validate_page_tags(tags, bt, exp, lens, S)
        got_verdict = verdict_t.cpu().numpy()
        assert np.array_equal(got_verdict, want_verdict)
        # block 0 of request 2 was freed but not handed out again (its tag is
        # unchanged); block 1 went to request 5 and fails first
        assert got_verdict.tolist() == [0, 0, 2, 0, 0, 0]
    ref = oracle.paged_decode_attn(q, okc, ovc, ks, vs, bt, lens, num_kv_heads=HKV,
                                   head_dim_v=D, page_size=S, num_pages=P, kv_dtype=1,
                                   scale_mode=1, v_in_k=False, sm_scale=cfg.sm_scale,
                                   verdict=want_verdict)
    got = out.cpu().numpy()
    if track:
        assert np.all(got[STALE] == 0)
    assert_attn_close(got, ref, f"library pool step (tracking {track})")
