"""The C ABI without a GPU: libpda.so loads, exports every function that
include/pda.h declares, and rejects bad arguments with the documented status
codes before anything is enqueued (no call here reaches a kernel launch)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


def declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(",
                       text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "defined")))


@pytest.fixture(scope="module")
def pda():
    import decode_attention_fp8_write_amd as m
    m.load()
    return m


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(["kv_write_fp8", "kv_write_bf16", "kv_transcode_bf16_to_fp8",
                            "kv_write_check",
                            "pda_pool_create", "pda_pool_destroy", "pda_pool_alloc",
                            "pda_pool_free", "pda_pool_tags", "pda_pool_num_free",
                            "pda_hbm_read_probe", "pda_hbm_read_probe_sink_words",
                            "int4_gemv_bf16", "validate_page_tags",
                            "paged_decode_attn_workspace_bytes", "paged_decode_attn",
                            "paged_decode_attn_noalloc",
                            "paged_decode_attn_noalloc_scratch_bytes", "pda_status_string"])


def test_library_exports_every_declared_symbol(pda):
    lib = pda.load()
    for name in declared_functions():
        assert hasattr(lib, name), f"libpda.so does not export {name}"
    assert set(pda.EXPORTS) == set(declared_functions())


def test_status_strings(pda):
    assert pda.status_string(pda.PDA_OK) == "ok"
    assert pda.status_string(pda.PDA_ERR_INVALID_ARG) == "invalid argument"
    assert pda.status_string(pda.PDA_ERR_UNSUPPORTED) == "unsupported shape or dtype"
    assert pda.status_string(pda.PDA_ERR_LAUNCH) == "kernel launch failed"
    assert pda.status_string(pda.PDA_ERR_WORKSPACE) == "workspace too small"
    assert "scratch" in pda.status_string(pda.PDA_ERR_SCRATCH)
    assert pda.status_string(99) == "unknown status"


def _shape(pda, **kw):
    base = dict(num_seqs=64, num_q_heads=64, num_kv_heads=8, head_dim_qk=128, head_dim_v=128,
                page_size=16, num_pages=32768, max_blocks_per_seq=512,
                kv_dtype=pda.KV_FP8_E4M3, scale_mode=pda.SCALE_PER_HEAD, split_tokens=512,
                sm_scale=0.08838834764831845)
    base.update(kw)
    return pda.make_shape(**base)


def test_workspace_sizes(pda):
    # 64 seqs x 4 units (of four 512-token chunks) x 8 kv heads, each
    # partial 8 rows x (128 + 2) fp32, after a 256-byte-aligned header of
    # (64 + 65) ints
    sh = _shape(pda)
    assert pda.paged_decode_attn_workspace_bytes(sh, 8192) == 768 + 64 * 4 * 8 * 8 * 130 * 4
    # a ragged chunk count rounds up to whole units: 8193 tokens = 17 chunks
    assert pda.paged_decode_attn_workspace_bytes(sh, 8193) == 768 + 64 * 5 * 8 * 8 * 130 * 4
    # invalid shapes give 0
    for bad in (dict(num_q_heads=60), dict(num_kv_heads=0), dict(page_size=0),
                dict(split_tokens=100), dict(kv_dtype=7), dict(sm_scale=float("nan"))):
        assert pda.paged_decode_attn_workspace_bytes(_shape(pda, **bad), 8192) == 0, bad
    assert pda.paged_decode_attn_workspace_bytes(sh, -1) == 0
    # latent path: one partial of 128 x (512 + 4) fp32 per (workgroup + sequence)
    lat_kw = dict(num_q_heads=128, num_kv_heads=1, head_dim_qk=576, head_dim_v=512,
                  page_size=64, kv_dtype=pda.KV_FP8_E4M3, scale_mode=pda.SCALE_PER_TOKEN,
                  v_in_k=True, split_tokens=0, sm_scale=1.0 / 24)
    lat = _shape(pda, **lat_kw)
    n = pda.paged_decode_attn_workspace_bytes(lat, 32768)
    slot = 128 * 516 * 4
    assert n > 0 and (n - 768) % slot == 0 and (n - 768) // slot > 64
    # the latent kernel takes 32, 64, 96 or 128 heads and at most 2048 sequences
    for hq in (32, 64, 96):
        assert pda.paged_decode_attn_workspace_bytes(_shape(pda, **{**lat_kw, "num_q_heads": hq}),
                                                     32768) > 0, hq
    for bad in (dict(num_q_heads=48), dict(num_q_heads=160), dict(num_seqs=2049)):
        assert pda.paged_decode_attn_workspace_bytes(_shape(pda, **{**lat_kw, **bad}), 32768) == 0, bad
    assert pda.paged_decode_attn_workspace_bytes(_shape(pda, **{**lat_kw, "num_seqs": 2048}),
                                                 32768) > 0


def test_argument_checks_return_before_launch(pda):
    lib = pda.load()
    null = None
    sh = _shape(pda)
    # null device pointers
    st = lib.paged_decode_attn(ctypes.byref(sh), null, null, null, null, null, null, null, 8192,
                               null, null, 0, null, null)
    assert st == pda.PDA_ERR_INVALID_ARG
    # unsupported head dim on an otherwise valid shape
    sh2 = _shape(pda, head_dim_qk=96, head_dim_v=96)
    fake = ctypes.c_void_p(256)
    st = lib.paged_decode_attn(ctypes.byref(sh2), fake, fake, fake, fake, fake, fake, fake, 8192,
                               null, fake, 1 << 20, fake, null)
    assert st == pda.PDA_ERR_UNSUPPORTED
    # workspace too small
    st = lib.paged_decode_attn(ctypes.byref(sh), fake, fake, fake, fake, fake, fake, fake, 8192,
                               null, fake, 16, fake, null)
    assert st == pda.PDA_ERR_WORKSPACE
    # kv_write: bad scale mode, per-token on a non-latent cache, bad sizes
    st = lib.kv_write_fp8(fake, fake, fake, 4, 8, 128, 128, 16, 64, 7, fake, fake, null, fake,
                          fake, null)
    assert st == pda.PDA_ERR_INVALID_ARG
    st = lib.kv_write_fp8(fake, fake, fake, 4, 8, 128, 128, 16, 64, pda.SCALE_PER_TOKEN, null,
                          null, fake, fake, fake, null)
    assert st == pda.PDA_ERR_UNSUPPORTED
    st = lib.kv_write_bf16(fake, fake, fake, -1, 8, 128, 128, 16, 64, fake, fake, null)
    assert st == pda.PDA_ERR_INVALID_ARG
    st = lib.kv_write_bf16(fake, fake, fake, 4, 8, 100, 128, 16, 64, fake, fake, null)
    assert st == pda.PDA_ERR_UNSUPPORTED
    # zero tokens / zero sequences are valid no-ops
    assert lib.kv_write_bf16(fake, fake, fake, 0, 8, 128, 128, 16, 64, fake, fake, null) == 0
    assert lib.validate_page_tags(null, 64, null, null, 16, null, 0, 16, null, null) == 0
    # validate: non-positive sizes, null pointers
    assert lib.validate_page_tags(fake, 0, fake, fake, 16, fake, 4, 16, fake, null) == \
        pda.PDA_ERR_INVALID_ARG
    assert lib.validate_page_tags(null, 64, fake, fake, 16, fake, 4, 16, fake, null) == \
        pda.PDA_ERR_INVALID_ARG


def test_write_check_argument_checks(pda):
    """kv_write_check refuses what either call it replaces refuses, before
    anything is launched."""
    lib = pda.load()
    null = None
    fake = ctypes.c_void_p(256)

    def call(T=4, dtype=None, mode=None, ks=fake, vs=fake, ts=null, tags=fake, B=4, ver=fake,
             mb=16, dk=128):
        dtype = pda.KV_FP8_E4M3 if dtype is None else dtype
        mode = pda.SCALE_PER_HEAD if mode is None else mode
        return lib.kv_write_check(fake, fake, fake, T, 8, dk, 128, 16, 64, dtype, mode, ks, vs,
                                  ts, fake, fake, tags, fake, fake, mb, fake, B, ver, null)

    assert call(dtype=7) == pda.PDA_ERR_INVALID_ARG                 # unknown cache dtype
    assert call(mode=7) == pda.PDA_ERR_INVALID_ARG                  # unknown scale mode
    assert call(dtype=pda.KV_BF16) == pda.PDA_ERR_INVALID_ARG       # BF16 takes no scales
    assert call(mode=pda.SCALE_PER_TOKEN, ks=null, vs=null, ts=fake) == pda.PDA_ERR_UNSUPPORTED
    assert call(dk=100) == pda.PDA_ERR_UNSUPPORTED                  # the write's shape rules
    assert call(T=-1) == pda.PDA_ERR_INVALID_ARG
    assert call(B=-1) == pda.PDA_ERR_INVALID_ARG                    # the check's sizes
    assert call(mb=0) == pda.PDA_ERR_INVALID_ARG
    assert call(tags=null) == pda.PDA_ERR_INVALID_ARG               # the check's pointers
    assert call(ver=null) == pda.PDA_ERR_INVALID_ARG
    # nothing to do: a no-op; sequences only need no write pointers checked
    assert call(T=0, B=0) == pda.PDA_OK
    assert call(B=0, tags=null, ver=null, T=0) == pda.PDA_OK


def test_transcode_argument_checks(pda):
    lib = pda.load()
    null = None
    fake = ctypes.c_void_p(256)
    # (k_src, v_src, src, dst, valid, n, hkv, dk, dv, S, Ps, Pd, mode, ks, vs, ts, kd, vd, stream)
    ok = [fake, fake, fake, fake, fake, 4, 8, 128, 128, 16, 64, 64, pda.SCALE_PER_HEAD, fake,
          fake, null, fake, fake, null]

    def call(**kw):
        args = list(ok)
        names = ["k_src", "v_src", "src", "dst", "valid", "n", "hkv", "dk", "dv", "S", "Ps",
                 "Pd", "mode", "ks", "vs", "ts", "kd", "vd", "stream"]
        for k, v in kw.items():
            args[names.index(k)] = v
        return lib.kv_transcode_bf16_to_fp8(*args)

    assert call(n=0) == pda.PDA_OK                          # nothing to do
    assert call(n=-1) == pda.PDA_ERR_INVALID_ARG
    assert call(src=null) == pda.PDA_ERR_INVALID_ARG
    assert call(v_src=null) == pda.PDA_ERR_INVALID_ARG      # latent source, non-latent dest
    assert call(dk=100) == pda.PDA_ERR_UNSUPPORTED
    assert call(S=15) == pda.PDA_ERR_UNSUPPORTED
    assert call(mode=7) == pda.PDA_ERR_INVALID_ARG
    assert call(ts=fake) == pda.PDA_ERR_INVALID_ARG         # per-head takes no token scales
    assert call(mode=pda.SCALE_PER_TOKEN, ks=null, vs=null, ts=fake) == \
        pda.PDA_ERR_UNSUPPORTED                             # per-token needs a latent cache
    assert call(k_src=ctypes.c_void_p(264)) == pda.PDA_ERR_INVALID_ARG   # misaligned
    assert call(Ps=0) == pda.PDA_ERR_INVALID_ARG


def test_read_probe_argument_checks(pda):
    lib = pda.load()
    fake = ctypes.c_void_p(256)
    null = None
    E = pda.PDA_ERR_INVALID_ARG
    assert lib.pda_hbm_read_probe(null, 4096, 0, fake, null) == E
    assert lib.pda_hbm_read_probe(fake, 4096, 0, null, null) == E
    assert lib.pda_hbm_read_probe(ctypes.c_void_p(264), 4096, 0, fake, null) == E   # misaligned
    assert lib.pda_hbm_read_probe(fake, 4100, 0, fake, null) == E      # not whole 16-byte words
    assert lib.pda_hbm_read_probe(fake, 8192, 3000, fake, null) == E   # chunk not a power of two
    assert lib.pda_hbm_read_probe(fake, 8192, 128, fake, null) == E    # chunk too small
    assert lib.pda_hbm_read_probe(fake, 3 * 2048, 2048, fake, null) == E   # 3 chunks


def test_int4_gemv_argument_checks(pda):
    lib = pda.load()
    f = ctypes.c_void_p(4096)
    null = None
    E, U, OK = pda.PDA_ERR_INVALID_ARG, pda.PDA_ERR_UNSUPPORTED, pda.PDA_OK
    g = lib.int4_gemv_bf16
    assert g(f, f, f, -1, 16, 128, 128, f, null) == E
    assert g(f, f, f, 1, -16, 128, 128, f, null) == E
    assert g(f, f, f, 1, 16, 128, 64, f, null) == U          # group other than 128
    assert g(f, f, f, 1, 16, 200, 128, f, null) == U         # k not a multiple of 128
    assert g(f, f, f, 1, 16, 0, 128, f, null) == U           # k == 0 with work to do
    assert g(null, null, null, 0, 16, 128, 128, null, null) == OK   # nothing to do
    assert g(null, null, null, 4, 0, 128, 128, null, null) == OK
    assert g(null, f, f, 1, 16, 128, 128, f, null) == E
    assert g(f, f, f, 1, 16, 128, 128, null, null) == E
    assert g(ctypes.c_void_p(4104), f, f, 1, 16, 128, 128, f, null) == E   # x not 16-aligned
    assert g(f, ctypes.c_void_p(4100), f, 1, 16, 128, 128, f, null) == E   # w not 16-aligned
    assert g(f, ctypes.c_void_p(4104), f, 1, 16, 128, 128, f, null) == E
    assert g(f, f, ctypes.c_void_p(4097), 1, 16, 128, 128, f, null) == E   # scale odd
    assert g(f, f, f, 1, 16, 128, 128, ctypes.c_void_p(4098), null) == E   # y not 4-aligned
    assert g(f, f, f, 2097121, 16, 128, 128, f, null) == U   # too many tokens for the grid


def test_noalloc_host_checks(pda):
    """The allocation-free entry point: its scratch size, and the argument
    and size checks it makes on the host before touching any device."""
    lib = pda.load()
    assert pda.paged_decode_attn_noalloc_scratch_bytes() == 96 << 20
    fake = ctypes.c_void_p(256)
    sh = _shape(pda)
    st = lib.paged_decode_attn_noalloc(ctypes.byref(sh), None, fake, fake, fake, fake, fake,
                                       fake, 8192, None, fake, None)
    assert st == pda.PDA_ERR_INVALID_ARG
    st = lib.paged_decode_attn_noalloc(ctypes.byref(sh), fake, fake, fake, fake, fake, fake,
                                       fake, -1, None, fake, None)
    assert st == pda.PDA_ERR_INVALID_ARG
    # 16384 sequences x 8 kv heads need 545 MB of partials even at one unit
    # per (sequence, kv head)
    big = _shape(pda, num_seqs=16384, split_tokens=0)
    st = lib.paged_decode_attn_noalloc(ctypes.byref(big), fake, fake, fake, fake, fake, fake,
                                       fake, 8192, None, fake, None)
    assert st == pda.PDA_ERR_SCRATCH
    # zero sequences: nothing to do
    st = lib.paged_decode_attn_noalloc(ctypes.byref(_shape(pda, num_seqs=0)), None, None,
                                       None, None, None, None, None, 0, None, None, None)
    assert st == pda.PDA_OK
