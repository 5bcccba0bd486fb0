"""GPU parity of paged_decode_attn (VALU path, GQA groups below 16 rows)
against the oracle, on small seeded problems that span several 64-token
blocks, several split-K chunks and ragged tails (fixed shapes and eight
seeded random ones over G, kv heads, page size and split), plus the method's edge
cases: aborted sequences (verdict != 0) read nothing and return zeros, the
no-op tracker (verdict NULL) matches an all-clear verdict bit for bit, a
physical page permutation leaves the output bit-identical, poisoned pages
and tail slots never leak into the result, and length 0 gives zeros.

Tolerance: max-abs 2e-3 and rel-L2 1e-3 against the fp64 oracle.
"""
import math

import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_attn_close, log
from helpers import oracle_attn, oracle_caches, slots_of, small_problem

pytestmark = pytest.mark.gpu


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


class GpuProblem:
    """Caches of a small problem written by the GPU kv_write kernels."""

    def __init__(self, gpu, pr, poison=None):
        self.gpu, self.pr = gpu, pr
        P, S, hkv, dk, dv = pr["P"], pr["S"], pr["hkv"], pr["dk"], pr["dv"]
        fp8 = pr["kv_dtype"] == synth.KV_FP8
        fill = synth.poison_value(pr["kv_dtype"]) if poison is None else poison
        if fp8:
            self.kc = torch.full((P * hkv * S * dk,), fill, dtype=torch.uint8, device="cuda")
            self.vc = torch.full((P * hkv * S * dv,), fill, dtype=torch.uint8, device="cuda")
            self.ks, self.vs = _dev(pr["k_scale"]), _dev(pr["v_scale"])
        else:
            f = fill - 0x10000 if fill >= 0x8000 else fill
            self.kc = torch.full((P * hkv * S * dk,), f, dtype=torch.int16, device="cuda")
            self.vc = torch.full((P * hkv * S * dv,), f, dtype=torch.int16, device="cuda")
            self.ks = self.vs = None
        for s, l in enumerate(pr["lens"]):
            if l == 0:
                continue
            slots = _dev(slots_of(pr["bt"][s], S, int(l)))
            k, v = _dev(pr["ks"][s]), _dev(pr["vs"][s])
            if fp8:
                gpu.kv_write_fp8(k, v, slots, self.kc, self.vc, page_size=S, num_pages=P,
                                 k_scale=self.ks, v_scale=self.vs)
            else:
                gpu.kv_write_bf16(k, v, slots, self.kc, self.vc, page_size=S, num_pages=P)
        self.q = _dev(pr["q"])

    def attend(self, bt=None, lens=None, verdict=None, split=0, ws_bytes=None,
               max_seq_len=None):
        gpu, pr = self.gpu, self.pr
        bt = pr["bt"] if bt is None else bt
        lens = pr["lens"] if lens is None else lens
        B = len(lens)
        fp8 = pr["kv_dtype"] == synth.KV_FP8
        shape = gpu.make_shape(
            num_seqs=B, num_q_heads=pr["hq"], num_kv_heads=pr["hkv"], head_dim_qk=pr["dk"],
            head_dim_v=pr["dv"], page_size=pr["S"], num_pages=pr["P"],
            max_blocks_per_seq=bt.shape[1],
            kv_dtype=gpu.KV_FP8_E4M3 if fp8 else gpu.KV_BF16,
            scale_mode=gpu.SCALE_PER_HEAD if fp8 else gpu.SCALE_NONE,
            split_tokens=split, sm_scale=pr["sm_scale"])
        msl = int(max(0, np.max(lens))) if max_seq_len is None else max_seq_len
        need = gpu.paged_decode_attn_workspace_bytes(shape, msl)
        ws = torch.empty(need if ws_bytes is None else ws_bytes, dtype=torch.uint8,
                         device="cuda")
        ws.fill_(0xFF)
        out = torch.full((B, pr["hq"], pr["dv"]), 7.0, dtype=torch.float32, device="cuda")
        gpu.paged_decode_attn(shape, self.q, self.kc, self.vc, self.ks, self.vs, _dev(bt),
                              _dev(np.asarray(lens, np.int32)), msl,
                              None if verdict is None else _dev(np.asarray(verdict, np.int32)),
                              ws, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()


CASES = [
    # (lens, hq, hkv, S, split)
    ([17, 64, 100, 255], 8, 2, 16, 0),           # workload-1 shape
    ([1, 63, 64, 65, 127, 129, 700], 16, 2, 16, 64),
    ([1000, 1537, 2049], 64, 8, 16, 512),
    ([300, 5, 1024], 8, 8, 16, 128),              # G = 1
    ([333, 77, 64], 8, 4, 32, 64),                # G = 2, S = 32
    ([1200, 65, 3], 16, 4, 64, 128),              # G = 4, S = 64
    ([4097, 2], 8, 1, 16, 0),                     # G = 8, one kv head
]


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_small_parity(gpu, case, kv_dtype):
    lens, hq, hkv, S, split = CASES[case]
    log(f"attn small case {case} dtype {kv_dtype}: lens {lens} hq {hq} hkv {hkv} S {S} split {split}")
    pr = small_problem(100 + case, lens, hq, hkv, 128, 128, S, kv_dtype)
    kc, vc, ts = oracle_caches(pr)
    ref = oracle_attn(pr, kc, vc, ts)
    g = GpuProblem(gpu, pr)
    got = g.attend(split=split)
    assert_attn_close(got, ref, f"case {case}")
    # deterministic: a second run is bit-identical
    assert np.array_equal(got, g.attend(split=split))


def _random_case(i):
    """Seeded random shape i for the vector-ALU path: G in {1, 2, 4, 8},
    1-8 kv heads, pages of 16, 32 or 64 tokens, split chunks of 0 (automatic)
    or 64-1024 tokens, 1-10 sequences of 1-2999 tokens (one of 3000-9999 in
    about a third of the cases)."""
    rng = np.random.default_rng(7000 + i)
    G = int(rng.choice([1, 2, 4, 8]))
    hkv = int(rng.choice([1, 2, 4, 8]))
    S = int(rng.choice([16, 32, 64]))
    split = int(rng.choice([0, 64, 128, 192, 512, 1024]))
    B = int(rng.integers(1, 11))
    lens = [int(x) for x in rng.integers(1, 3000, B)]
    if rng.random() < 0.35:
        lens[int(rng.integers(0, B))] = int(rng.integers(3000, 10000))
    return lens, G * hkv, hkv, S, split, int(rng.integers(0, 1 << 30))


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
@pytest.mark.parametrize("i", range(8))
def test_random_shapes(gpu, i, kv_dtype):
    lens, hq, hkv, S, split, seed = _random_case(i)
    log(f"attn random case {i} dtype {kv_dtype}: seed {seed} lens {lens} hq {hq} hkv {hkv} "
        f"S {S} split {split}")
    pr = small_problem(seed, lens, hq, hkv, 128, 128, S, kv_dtype)
    kc, vc, ts = oracle_caches(pr)
    ref = oracle_attn(pr, kc, vc, ts)
    g = GpuProblem(gpu, pr)
    got = g.attend(split=split)
    assert_attn_close(got, ref, f"random case {i}")
    assert np.array_equal(got, g.attend(split=split))


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
def test_outlier_channels(gpu, kv_dtype):
    """K with 6 of 128 channels scaled by 20 (the quantisation stress of the
    64 x 8192 workload) at a reduced length."""
    log(f"attn outliers dtype {kv_dtype}")
    pr = small_problem(7, [2000, 1500], 64, 8, 128, 128, 16, kv_dtype)
    rng = np.random.default_rng(8)
    for s in range(2):
        k = synth.bf16_to_f32(pr["ks"][s]).copy()
        for h in range(8):
            ch = rng.choice(128, 6, replace=False)
            k[:, h, ch] *= 20
        pr["ks"][s] = synth.bf16_from_f32(k)
    if kv_dtype == synth.KV_FP8:
        kam = np.max([np.abs(synth.bf16_to_f32(k)).max(axis=(0, 2)) for k in pr["ks"]], axis=0)
        pr["k_scale"] = (kam / np.float32(448)).astype(np.float32)
    kc, vc, ts = oracle_caches(pr)
    ref = oracle_attn(pr, kc, vc, ts)
    got = GpuProblem(gpu, pr).attend(split=512)
    assert_attn_close(got, ref, "outliers")


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
def test_abort_noop_and_permutation(gpu, kv_dtype):
    log(f"attn abort/no-op/permutation dtype {kv_dtype}")
    pr = small_problem(21, [130, 500, 64, 900], 16, 2, 128, 128, 16, kv_dtype, num_pages=120)
    kc, vc, ts = oracle_caches(pr)
    g = GpuProblem(gpu, pr)
    free = g.attend(split=128)
    allclear = g.attend(split=128, verdict=[0, 0, 0, 0])
    assert np.array_equal(free, allclear)
    ver = [0, 4, 0, -1]
    got = g.attend(split=128, verdict=ver)
    ref = oracle_attn(pr, kc, vc, ts, verdict=np.array(ver, np.int32))
    assert np.all(got[1] == 0) and np.all(got[3] == 0)
    assert np.array_equal(got[0], free[0]) and np.array_equal(got[2], free[2])
    assert_attn_close(got, ref, "abort")
    # a different physical placement of the same pages: bit-identical output
    rng = np.random.default_rng(5)
    perm = rng.permutation(pr["P"])
    pr2 = dict(pr)
    bt2 = pr["bt"].copy()
    bt2[bt2 >= 0] = perm[bt2[bt2 >= 0]]
    pr2["bt"] = bt2
    moved = GpuProblem(gpu, pr2).attend(split=128)
    assert np.array_equal(moved, free)


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
@pytest.mark.parametrize("poison", ["nan", "max"])
def test_poison_never_read(gpu, kv_dtype, poison):
    """Unused pages, tail slots past each length and every page of aborted
    sequences hold NaN codes (or the largest finite code); the result must
    still match the oracle, which never reads them."""
    log(f"attn poison {poison} dtype {kv_dtype}")
    fp8 = kv_dtype == synth.KV_FP8
    if poison == "nan":
        fill = synth.poison_value(kv_dtype)
    else:
        fill = 0x7E if fp8 else 0x7F7F
    pr = small_problem(31, [17, 64, 100, 255, 1], 8, 2, 128, 128, 16, kv_dtype, num_pages=64)
    kc, vc, ts = oracle_caches(pr, fill=fill)
    g = GpuProblem(gpu, pr, poison=fill)
    # aborted sequence 2: overwrite its pages with poison too
    S = 16
    pages2 = pr["bt"][2, :-(-100 // S)]
    pe = 2 * S * 128
    for p in pages2:
        g.kc[p * pe:(p + 1) * pe] = fill if fp8 else (fill - 0x10000 if fill >= 0x8000 else fill)
        g.vc[p * pe:(p + 1) * pe] = fill if fp8 else (fill - 0x10000 if fill >= 0x8000 else fill)
    ver = np.array([0, 0, 3, 0, 0], np.int32)
    for split in (0, 64):
        got = g.attend(verdict=ver, split=split)
        ref = oracle_attn(pr, kc, vc, ts, verdict=ver)
        assert np.isfinite(got).all()
        assert np.all(got[2] == 0)
        assert_attn_close(got, ref, f"poison {poison} split {split}")


def test_edge_rows(gpu):
    log("attn edge rows")
    pr = small_problem(41, [0, 20, 40, 33, 150], 8, 2, 128, 128, 16, synth.KV_FP8)
    kc, vc, ts = oracle_caches(pr)
    g = GpuProblem(gpu, pr)
    bt = pr["bt"].copy()
    bt[3, 1] = pr["P"]                 # out-of-range page id
    bt[4, 9] = -7                      # negative page id, last block
    lens = pr["lens"].copy()
    lens[2] = bt.shape[1] * 16 + 1     # longer than the block table
    got = g.attend(bt=bt, lens=lens, max_seq_len=150)
    ref = oracle_attn(pr, kc, vc, ts, bt=bt, lens=lens)
    assert np.all(got[0] == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3])) and np.all(np.isnan(got[4]))
    assert_attn_close(got[1], ref[1], "edge row 1")
    # under a verdict from the tracker the same rows are aborts (zeros)
    ver = np.array([0, 0, -1, 2, 10], np.int32)
    got = g.attend(bt=bt, lens=lens, verdict=ver, max_seq_len=150)
    assert np.all(got[2:] == 0) and np.all(got[0] == 0)
    assert_attn_close(got[1], ref[1], "edge row 1 with verdict")
    # all sequences empty
    got = g.attend(lens=np.zeros(5, np.int32), max_seq_len=0)
    assert np.all(got == 0)


def test_small_workspace_widens_chunks(gpu):
    log("attn small workspace")
    pr = small_problem(51, [3000, 100, 2500], 16, 2, 128, 128, 16, synth.KV_FP8)
    kc, vc, ts = oracle_caches(pr)
    ref = oracle_attn(pr, kc, vc, ts)
    g = GpuProblem(gpu, pr)
    full = g.attend(split=64)
    # room for one unit partial per (sequence, kv head) only
    hdr = 256 * (-(-((64 + 3 + 1) * 4) // 256))
    minimal = hdr + 3 * 2 * 8 * 130 * 4
    tight = g.attend(split=64, ws_bytes=minimal)
    assert_attn_close(full, ref, "full workspace")
    assert_attn_close(tight, ref, "minimal workspace")
    with pytest.raises(g.gpu.PdaError):
        g.attend(split=64, ws_bytes=minimal - 4)


def test_workload1_end_to_end(gpu):
    """Workload 1 as one decode step: write, validate (one injected mismatch
    aborts its sequence), attend; compared with the oracle on every row."""
    log("workload 1 end to end")
    from synth import device as workload
    from gpu_helpers import oracle_attn_subset, oracle_subset
    import oracle
    b = synth.make_batch(1)
    data = [b.kv(s) for s in range(b.B)]
    ver_ref = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags,
                                        b.seq_lens, 16)
    for kv_dtype in (synth.KV_FP8, synth.KV_BF16):
        db = workload.build(b, kv_dtype, data=data)
        db.alloc_workspace()
        db.validate()
        db.attend()
        torch.cuda.synchronize()
        assert np.array_equal(db.verdict.cpu().numpy(), ver_ref)
        sub = oracle_subset(b, data, list(range(b.B)), kv_dtype, db.host_scales)
        ref = oracle_attn_subset(b, sub, kv_dtype, db.host_scales, verdict=ver_ref)
        got = db.out.cpu().numpy()
        assert_attn_close(got, ref, f"workload 1 dtype {kv_dtype}")
        assert np.all(got[ver_ref != 0] == 0)


@pytest.mark.parametrize("kv_dtype", [synth.KV_FP8, synth.KV_BF16])
def test_many_short_sequences(gpu, kv_dtype):
    """The largest batch the vector-ALU path takes: 16384 sequences of 1 to
    48 tokens with the 64 x 8192 workload's heads (the per-sequence slot
    prefix then needs over 64 KB of LDS per workgroup), every row compared.
    K/V come from one seeded stream split by sequence (a per-sequence stream
    for 16384 sequences costs more host time than the test itself)."""
    import oracle
    from synth import device as workload
    from oracle.harness import oracle_attn_full, oracle_full_cache
    log(f"16384 short sequences, dtype {kv_dtype}")
    rng = np.random.default_rng(16384)
    lens = rng.integers(1, 49, size=16384)
    b = synth.make_batch(3, lens=lens)
    cfg = b.cfg
    T = int(lens.sum())
    k = synth.bf16_from_f32(rng.standard_normal((T, cfg.num_kv_heads, cfg.head_dim_qk),
                                                dtype=np.float32))
    v = synth.bf16_from_f32(rng.standard_normal((T, cfg.num_kv_heads, cfg.head_dim_v),
                                                dtype=np.float32))
    cut = np.concatenate([[0], np.cumsum(lens)])
    data = [(k[cut[s]:cut[s + 1]], v[cut[s]:cut[s + 1]]) for s in range(b.B)]
    db = workload.build(b, kv_dtype, data=data)
    db.alloc_workspace(split_tokens=0)
    db.step(use_verdict=True)
    torch.cuda.synchronize()
    verdict = db.verdict.cpu().numpy()
    assert np.all(verdict == 0)
    got = db.out.cpu().numpy()
    kc, vc, ts = oracle_full_cache(b, data, kv_dtype, db.host_scales)
    elt = np.uint8 if kv_dtype == synth.KV_FP8 else np.uint16
    assert np.array_equal(db.k_cache.cpu().numpy().view(elt), kc)
    assert np.array_equal(db.v_cache.cpu().numpy().view(elt), vc)
    want = oracle.validate_page_tags(b.page_tags, b.block_table, b.expected_tags,
                                     b.seq_lens, cfg.page_size)
    assert np.array_equal(verdict, want)
    ref = oracle_attn_full(b, kc, vc, ts, kv_dtype, db.host_scales, verdict)
    assert_attn_close(got, ref, f"16384 sequences dtype {kv_dtype}")
