"""The host page pool and tag tracker: the oracle pool pinned by the
properties the pages give the tags (a page handed out again carries a new
tag; the tags of pages in use are distinct; the no-op tracker stamps
nothing) and by the free-stack order, cross-checked against the input
generator's pool; then libpda.so's native pool (pda_pool_*) compared with
the oracle on long seeded operation sequences, invalid operations included.
Host code only: no GPU."""
import numpy as np
import pytest

import oracle
import synth
from oracle.pool import OraclePagePool


def test_oracle_pool_properties():
    pool = OraclePagePool(8, initial_order=[3, 1, 4, 0, 5, 2, 7, 6], tag_start=10)
    pages, tags = pool.alloc(3)
    assert pages == [3, 1, 4] and tags == [11, 12, 13]
    pool.free([1, 3])                     # pushed in order: 3 is handed out first
    pages2, tags2 = pool.alloc(2)
    assert pages2 == [3, 1] and tags2 == [14, 15]
    in_use = [4, 3, 1]
    assert len(set(pool.tags[p] for p in in_use)) == 3
    # exhaustion: nothing changes
    before = (list(pool.free_stack), list(pool.tags), pool.counter)
    with pytest.raises(MemoryError):
        pool.alloc(6)
    assert (list(pool.free_stack), list(pool.tags), pool.counter) == before
    # invalid frees: nothing changes
    for bad in ([0], [9], [-1], [4, 4], [4, 0]):
        with pytest.raises(ValueError):
            pool.free(bad)
        assert (list(pool.free_stack), list(pool.tags), pool.counter) == before
    # the counter wraps at 2^32
    w = OraclePagePool(4, tag_start=0xFFFFFFFE)
    assert w.alloc(3)[1] == [0xFFFFFFFF, 0, 1]
    # no-op tracker: no tag is stamped
    n = OraclePagePool(4, track_tags=False)
    p, t = n.alloc(4)
    assert t == [0, 0, 0, 0] and n.tags == [0, 0, 0, 0]


def test_oracle_pool_agrees_with_the_input_generator_pool():
    rng = np.random.default_rng(3)
    order_rng = np.random.default_rng(99)
    gen = synth.PagePool(64, np.random.default_rng(99))
    ref = OraclePagePool(64, initial_order=order_rng.permutation(64))
    live = []
    for _ in range(300):
        if live and rng.random() < 0.45:
            k = int(rng.integers(1, len(live) + 1))
            idx = sorted(rng.choice(len(live), k, replace=False).tolist(), reverse=True)
            out = [live.pop(i) for i in idx]
            gen.free(out)
            ref.free(out)
        else:
            n = int(rng.integers(0, min(8, ref.num_free) + 1))
            a = gen.alloc(n)
            b = ref.alloc(n)
            assert a[0].tolist() == b[0] and a[1].tolist() == b[1]
            live.extend(b[0])
        assert gen.tags.tolist() == ref.tags


def _next_op(rng, num_pages, live):
    """A seeded random operation: mostly valid allocs and frees of pages in
    use, with exhaustion, repeated ids and out-of-range ids mixed in."""
    r = rng.random()
    if r < 0.04:
        return "alloc", num_pages + 1                               # exhausted
    if r < 0.08 and live:
        p = live[int(rng.integers(len(live)))]
        return "free", [p, p]                                       # repeated
    if r < 0.10:
        return "free", [int(rng.integers(num_pages, 2 * num_pages))]   # out of range
    if live and r < 0.50:
        k = int(rng.integers(1, len(live) + 1))
        idx = rng.choice(len(live), k, replace=False)
        return "free", [live[i] for i in idx]
    return "alloc", int(rng.integers(0, 40))


@pytest.mark.parametrize("track", [True, False])
def test_native_pool_matches_the_oracle(track):
    import decode_attention_fp8_write_amd as pda
    P = 200
    order = np.random.default_rng(5).permutation(P)
    nat = pda.PagePool(P, initial_order=order, tag_start=0xFFFFFF00, track_tags=track)
    ref = OraclePagePool(P, initial_order=order, tag_start=0xFFFFFF00, track_tags=track)
    rng = np.random.default_rng(11 + track)
    live = []
    n_ok = n_err = 0
    for _ in range(4000):
        kind, arg = _next_op(rng, P, live)
        if kind == "alloc":
            try:
                want = ref.alloc(arg)
            except MemoryError:
                want = None
            if want is None:
                with pytest.raises(pda.PdaError) as e:
                    nat.alloc(arg)
                assert e.value.status == pda.PDA_ERR_POOL_EXHAUSTED
                n_err += 1
            else:
                got = nat.alloc(arg)
                assert got[0].tolist() == want[0] and got[1].tolist() == want[1]
                live.extend(want[0])
                n_ok += 1
        else:
            try:
                ref.free(arg)
                ok = True
            except ValueError:
                ok = False
            if ok:
                nat.free(arg)
                gone = set(arg)
                live = [p for p in live if p not in gone]
                n_ok += 1
            else:
                with pytest.raises(pda.PdaError) as e:
                    nat.free(arg)
                assert e.value.status == pda.PDA_ERR_INVALID_ARG
                n_err += 1
        assert nat.num_free == ref.num_free
        assert nat.tags().tolist() == ref.tags
    assert n_ok > 1000 and n_err > 100


def test_reallocated_pages_fail_the_tag_check():
    """Host story end to end: requests record the pages and tags the pool
    gave them; when a request's pages are freed and handed to another
    request, the batched check (here the oracle's) flags the stale request at
    its first reused block and passes the others."""
    import decode_attention_fp8_write_amd as pda
    S, P = 16, 32
    pool = pda.PagePool(P, initial_order=np.arange(P))
    lens = [40, 64, 33]
    tables, expected = [], []
    for l in lens:
        pages, tags = pool.alloc(-(-l // S))
        tables.append(pages)
        expected.append(tags)
    # request 1 is evicted; its pages go to a new request (reused first)
    pool.free(tables[1][::-1])
    newp, _ = pool.alloc(2)
    assert set(newp.tolist()) <= set(tables[1].tolist())
    mb = max(len(t) for t in tables)
    bt = np.full((3, mb), -1, np.int32)
    et = np.zeros((3, mb), np.uint32)
    for i, (t, e) in enumerate(zip(tables, expected)):
        bt[i, :len(t)] = t
        et[i, :len(e)] = e
    verdict = oracle.validate_page_tags(pool.tags(), bt, et, np.int32(lens), S)
    first_reused = min(int(np.where(tables[1] == p)[0][0]) for p in newp)
    assert verdict.tolist() == [0, first_reused + 1, 0]


@pytest.mark.parametrize("cid", [1, 2, 3, 4, 5])
def test_library_pool_replays_every_workload(cid):
    """Every workload's page bookkeeping (block tables, expected tags, page
    tags after injection), built once with the harness's pool and once with
    the library's pda_pool_* driven through the same seeded operations: the
    full-pool workload's six rounds of allocate/free churn included, the two
    agree exactly."""
    import decode_attention_fp8_write_amd as pda
    pda.load()
    a = synth.make_batch(cid)
    b = synth.make_batch(cid, pool_factory=lambda n, o: pda.PagePool(n, initial_order=o))
    assert np.array_equal(a.block_table, b.block_table)
    assert np.array_equal(a.expected_tags, b.expected_tags)
    assert np.array_equal(a.page_tags, b.page_tags)
    assert a.injected == b.injected
