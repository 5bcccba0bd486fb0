"""GPU parity of paged_decode_attn's latent path (one kv head of 576 FP8 dims
whose first 512 dims are the value, one scale per token, 32..128 query heads,
pages of 64 tokens; the MFMA kernel) against the oracle, on small seeded
problems spanning several pages, ragged last pages and several workgroup
ranges of the flat page split, plus aborted sequences, the no-op tracker,
a physical page permutation (bit-identical), poisoned slots (NaN codes and
NaN scales in every slot no sequence owns), empty / malformed rows and
eight seeded random shapes.

Tolerance: max-abs 2e-3 and rel-L2 1e-3 against the fp64 oracle.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_helpers import assert_attn_close, log
from helpers import oracle_attn, oracle_caches, slots_of, small_problem

pytestmark = pytest.mark.gpu

DK, DV, S = 576, 512, 64


def _dev(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).cuda()


class LatentProblem:
    """Cache of a small latent problem written by the GPU kv_write kernel."""

    def __init__(self, gpu, pr):
        self.gpu, self.pr = gpu, pr
        P = pr["P"]
        self.kc = torch.full((P * S * DK,), synth.FP8_POISON, dtype=torch.uint8, device="cuda")
        self.ts = torch.full((P * S,), float("nan"), dtype=torch.float32, device="cuda")
        for s, l in enumerate(pr["lens"]):
            if l == 0:
                continue
            slots = _dev(slots_of(pr["bt"][s], S, int(l)))
            gpu.kv_write_fp8(_dev(pr["ks"][s]), None, slots, self.kc, None, page_size=S,
                             num_pages=P, scale_mode=gpu.SCALE_PER_TOKEN, token_scale=self.ts)
        self.q = _dev(pr["q"])

    def attend(self, bt=None, lens=None, verdict=None, max_seq_len=None):
        gpu, pr = self.gpu, self.pr
        bt = pr["bt"] if bt is None else bt
        lens = pr["lens"] if lens is None else lens
        B = len(lens)
        shape = gpu.make_shape(
            num_seqs=B, num_q_heads=pr["hq"], num_kv_heads=1, head_dim_qk=DK, head_dim_v=DV,
            page_size=S, num_pages=pr["P"], max_blocks_per_seq=bt.shape[1],
            kv_dtype=gpu.KV_FP8_E4M3, scale_mode=gpu.SCALE_PER_TOKEN, v_in_k=True,
            sm_scale=pr["sm_scale"])
        msl = int(max(0, np.max(lens))) if max_seq_len is None else max_seq_len
        need = gpu.paged_decode_attn_workspace_bytes(shape, msl)
        assert need > 0
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        out = torch.full((B, pr["hq"], DV), 7.0, dtype=torch.float32, device="cuda")
        gpu.paged_decode_attn(shape, self.q, self.kc, None, self.ts, None, _dev(bt),
                              _dev(np.asarray(lens, np.int32)), msl,
                              None if verdict is None else _dev(np.asarray(verdict, np.int32)),
                              ws, out)
        torch.cuda.synchronize()
        return out.cpu().numpy()


CASES = [
    # (lens, hq)
    ([1, 63, 64, 65, 200], 128),
    ([1000, 3000, 129], 128),
    ([700, 64], 32),
    ([2048, 1, 333], 64),
    ([130, 95, 4000, 17, 64, 640], 96),
    # more pages (501) than workgroups (one per CU): fragments of several
    # pages, so every page after a fragment's first arrives by the copy
    # issued during the page before it
    ([20000, 9000, 3000], 64),
]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_latent_parity(gpu, case):
    lens, hq = CASES[case]
    log(f"latent case {case}: lens {lens} hq {hq}")
    pr = small_problem(300 + case, lens, hq, 1, DK, DV, S, synth.KV_FP8, latent=True)
    kc, vc, ts = oracle_caches(pr)
    ref = oracle_attn(pr, kc, vc, ts)
    g = LatentProblem(gpu, pr)
    # the GPU writer produced the same bytes and scales as the oracle's
    assert np.array_equal(g.kc.cpu().numpy(), kc)
    assert np.array_equal(g.ts.cpu().numpy().view(np.uint32), ts.view(np.uint32))
    got = g.attend()
    mx, rel = assert_attn_close(got, ref, f"latent case {case}")
    log(f"  max_abs {mx:.3e} rel_l2 {rel:.3e}")
    assert np.array_equal(got, g.attend()), "not deterministic"


def _random_case(i):
    """Seeded random latent problem i: 1-12 sequences of 1-3999 tokens, one
    of them 8000-19999 tokens in about a third of the cases (a sequence over
    many workgroups' fragments, merged in several chunks), 32-128 heads."""
    rng = np.random.default_rng(9000 + i)
    B = int(rng.integers(1, 13))
    lens = [int(x) for x in rng.integers(1, 4000, B)]
    if rng.random() < 0.35:
        lens[int(rng.integers(0, B))] = int(rng.integers(8000, 20000))
    return lens, int(rng.choice([32, 64, 96, 128])), int(rng.integers(0, 1 << 30))


@pytest.mark.parametrize("i", range(8))
def test_latent_random_shapes(gpu, i):
    lens, hq, seed = _random_case(i)
    log(f"latent random case {i}: seed {seed} hq {hq} lens {lens}")
    pr = small_problem(seed, lens, hq, 1, DK, DV, S, synth.KV_FP8, latent=True)
    kc, vc, ts = oracle_caches(pr)
    ref = oracle_attn(pr, kc, vc, ts)
    g = LatentProblem(gpu, pr)
    got = g.attend()
    mx, rel = assert_attn_close(got, ref, f"latent random case {i}")
    log(f"  max_abs {mx:.3e} rel_l2 {rel:.3e}")
    assert np.array_equal(got, g.attend()), "not deterministic"


def test_latent_abort_noop_permutation(gpu):
    log("latent abort / no-op / permutation")
    pr = small_problem(310, [500, 130, 2000, 64], 128, 1, DK, DV, S, synth.KV_FP8,
                       num_pages=60, latent=True)
    kc, vc, ts = oracle_caches(pr)
    g = LatentProblem(gpu, pr)
    free = g.attend()
    assert np.array_equal(free, g.attend(verdict=[0, 0, 0, 0]))
    ver = np.array([0, 2, 0, -1], np.int32)
    got = g.attend(verdict=ver)
    ref = oracle_attn(pr, kc, vc, ts, verdict=ver)
    assert np.all(got[1] == 0) and np.all(got[3] == 0)
    assert_attn_close(got, ref, "latent abort")
    # the flat page split depends on page counts only, not on page ids: a
    # different physical placement gives the same bits
    rng = np.random.default_rng(11)
    perm = rng.permutation(pr["P"])
    pr2 = dict(pr)
    bt2 = pr["bt"].copy()
    bt2[bt2 >= 0] = perm[bt2[bt2 >= 0]]
    pr2["bt"] = bt2
    moved = LatentProblem(gpu, pr2).attend()
    assert np.array_equal(moved, free)


def test_latent_edge_rows(gpu):
    log("latent edge rows")
    pr = small_problem(320, [0, 100, 70, 90, 300], 64, 1, DK, DV, S, synth.KV_FP8,
                       latent=True)
    kc, vc, ts = oracle_caches(pr)
    g = LatentProblem(gpu, pr)
    bt = pr["bt"].copy()
    bt[3, 1] = pr["P"]            # out-of-range page id
    lens = pr["lens"].copy()
    lens[2] = bt.shape[1] * S + 1  # longer than the block table
    got = g.attend(bt=bt, lens=lens, max_seq_len=300)
    ref = oracle_attn(pr, kc, vc, ts, bt=bt, lens=lens)
    assert np.all(got[0] == 0)
    assert np.all(np.isnan(got[2])) and np.all(np.isnan(got[3]))
    assert_attn_close(got[[1, 4]], ref[[1, 4]], "latent edge rows")
    got = g.attend(lens=np.zeros(5, np.int32), max_seq_len=0)
    assert np.all(got == 0)
