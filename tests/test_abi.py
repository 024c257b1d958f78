"""C-ABI checks that need no GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any HIP call."""
import ctypes
import os
import re
import subprocess

import pytest

import query_aware_sparse_min_amd as sa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")


def _lib():
    if not os.path.exists(sa.LIB_PATH):
        from query_aware_sparse_min_amd import build
        build.build()
    return sa.load()


def _declared():
    txt = open(HEADER).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z_0-9]+)\s*\(", txt)))


def test_header_declares_exactly_the_bound_exports():
    assert _declared() == sorted(sa.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in _declared():
        assert hasattr(lib, name), name
    out = subprocess.check_output(["nm", "-D", "--defined-only", sa.LIB_PATH], text=True)
    syms = {ln.split()[-1] for ln in out.splitlines() if ln.strip()}
    for name in _declared():
        assert name in syms, name


def test_library_links_no_oracle_code():
    out = subprocess.check_output(["nm", "-D", sa.LIB_PATH], text=True)
    assert "oracle_" not in out
    ldd = subprocess.check_output(["ldd", sa.LIB_PATH], text=True)
    assert "liboracle" not in ldd and "libsynth" not in ldd


def test_status_strings_and_version():
    _lib()
    assert sa.load().sa_version() >= 1
    assert sa.status_string(0) == "ok"
    for code in (-1, -2, -3, -4):
        assert sa.status_string(code) not in ("ok", "unknown status")
    assert sa.status_string(12345) == "unknown status"


FAKE = 0x10000  # a 16-byte-aligned non-null address; never dereferenced on these paths


def _kv(**kw):
    d = dict(k=FAKE, v=FAKE, k_scale=None, v_scale=None, dtype=sa.SA_BF16, num_pages=64,
             page_size=16, num_kv_heads=8, head_dim=128)
    d.update(kw)
    return sa.sa_kv_cache(**d)


def _seqs(**kw):
    d = dict(page_table=FAKE, seq_lens=FAKE, batch=2, max_pages=32)
    d.update(kw)
    return sa.sa_seqs(**d)


def _cfg(**kw):
    d = dict(mode=sa.SA_MODE_QUEST, unit_tokens=16, k_compete=6, n_head_forced=1,
             n_tail_forced=1, rank=16, proj=None, lse_scale=0.088)
    d.update(kw)
    return sa.sa_select_cfg(**d)


def _score(lib, kv, seqs, cfg, q=FAKE, qdt=sa.SA_BF16, hq=32, meta=FAKE, scores=FAKE):
    return lib.sa_score_pages(q, qdt, hq, ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(cfg),
                              meta, None, scores, None)


def test_sizes_are_host_side_and_consistent():
    lib = _lib()
    kv, seqs, cfg = _kv(), _seqs(), _cfg()
    assert lib.sa_meta_bytes(ctypes.byref(kv), ctypes.byref(cfg)) == 64 * 8 * 2 * 128 * 2
    assert lib.sa_meta_scale_bytes(ctypes.byref(kv), ctypes.byref(cfg)) == 0
    sals = _cfg(mode=sa.SA_MODE_SALS, unit_tokens=64, k_compete=32, n_head_forced=0,
                n_tail_forced=2, proj=FAKE)
    assert lib.sa_meta_bytes(ctypes.byref(kv), ctypes.byref(sals)) == 64 * 16 * 8 * 8
    assert lib.sa_meta_scale_bytes(ctypes.byref(kv), ctypes.byref(sals)) == 64 * 16 * 8 * 2
    assert lib.sa_max_units(ctypes.byref(seqs), ctypes.byref(cfg)) == 32
    assert lib.sa_max_units(ctypes.byref(seqs), ctypes.byref(sals)) == 8
    assert lib.sa_max_selected(ctypes.byref(seqs), ctypes.byref(cfg)) == 8
    assert lib.sa_max_selected(ctypes.byref(seqs), ctypes.byref(sals)) == 32  # clipped to max_pages
    assert lib.sa_decode_step_workspace_size(32, ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(cfg)) > 0
    assert lib.sa_attn_workspace_size(2, 32, 8, 32, 8) > 0
    assert lib.sa_attn_workspace_size(2, 30, 8, 32, 8) == 0  # group not integral
    assert lib.sa_attn_workspace_size(2, 24, 8, 32, 8) == 0  # G = 3 unsupported


@pytest.mark.parametrize("case,expect", [
    (dict(kv=dict(k=None)), sa.SA_ERR_INVALID_ARG),
    (dict(kv=dict(page_size=32)), sa.SA_ERR_UNSUPPORTED),
    (dict(kv=dict(head_dim=64)), sa.SA_ERR_UNSUPPORTED),
    (dict(kv=dict(dtype=7)), sa.SA_ERR_INVALID_ARG),
    (dict(kv=dict(k=FAKE + 4)), sa.SA_ERR_INVALID_ARG),
    (dict(kv=dict(dtype=sa.SA_I8)), sa.SA_ERR_INVALID_ARG),               # int8 without scales
    (dict(kv=dict(dtype=sa.SA_I8, k_scale=FAKE, v_scale=FAKE)), sa.SA_ERR_UNSUPPORTED),  # Quest on int8
    (dict(seqs=dict(batch=0)), sa.SA_ERR_INVALID_ARG),
    (dict(seqs=dict(seq_lens=None)), sa.SA_ERR_INVALID_ARG),
    (dict(cfg=dict(k_compete=-1)), sa.SA_ERR_INVALID_ARG),
    (dict(cfg=dict(k_compete=0, n_head_forced=0, n_tail_forced=0)), sa.SA_ERR_INVALID_ARG),
    (dict(cfg=dict(unit_tokens=24)), sa.SA_ERR_INVALID_ARG),
    (dict(cfg=dict(unit_tokens=32)), sa.SA_ERR_UNSUPPORTED),             # Quest units are pages
    (dict(cfg=dict(mode=9)), sa.SA_ERR_INVALID_ARG),
    (dict(cfg=dict(mode=sa.SA_MODE_SALS, unit_tokens=64)), sa.SA_ERR_INVALID_ARG),  # no projection
    (dict(cfg=dict(mode=sa.SA_MODE_SALS, unit_tokens=64, proj=FAKE, rank=8)), sa.SA_ERR_UNSUPPORTED),
    (dict(hq=30), sa.SA_ERR_INVALID_ARG),
    (dict(hq=24), sa.SA_ERR_UNSUPPORTED),
    (dict(qdt=sa.SA_I8), sa.SA_ERR_INVALID_ARG),
    (dict(q=None), sa.SA_ERR_INVALID_ARG),
    (dict(meta=None), sa.SA_ERR_INVALID_ARG),
    (dict(scores=None), sa.SA_ERR_INVALID_ARG),
])
def test_score_pages_rejects_bad_arguments(case, expect):
    lib = _lib()
    kv = _kv(**case.get("kv", {}))
    seqs = _seqs(**case.get("seqs", {}))
    cfg = _cfg(**case.get("cfg", {}))
    extra = {k: v for k, v in case.items() if k not in ("kv", "seqs", "cfg")}
    assert _score(lib, kv, seqs, cfg, **extra) == expect


def test_workspace_too_small_is_reported_before_launch():
    lib = _lib()
    kv, seqs, cfg = _kv(), _seqs(), _cfg()
    need = lib.sa_decode_step_workspace_size(32, ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(cfg))
    rc = lib.sa_decode_step(FAKE, sa.SA_BF16, 32, ctypes.byref(kv), ctypes.byref(seqs),
                            ctypes.byref(cfg), FAKE, None, 0.088, FAKE, None, None, FAKE, need - 1,
                            None)
    assert rc == sa.SA_ERR_WORKSPACE_TOO_SMALL
    need_a = lib.sa_attn_workspace_size(2, 32, 8, 32, 8)
    rc = lib.sa_sparse_decode_attn(FAKE, sa.SA_BF16, 32, ctypes.byref(kv), ctypes.byref(seqs), FAKE,
                                   FAKE, 8, 0.088, FAKE, FAKE, need_a - 1, None)
    assert rc == sa.SA_ERR_WORKSPACE_TOO_SMALL


def test_attention_argument_checks():
    lib = _lib()
    kv, seqs = _kv(), _seqs()
    call = lambda **kw: lib.sa_sparse_decode_attn(
        kw.get("q", FAKE), sa.SA_BF16, 32, ctypes.byref(kv), ctypes.byref(seqs), kw.get("sel", FAKE),
        kw.get("num", FAKE), kw.get("max_sel", 8), kw.get("scale", 0.088), kw.get("out", FAKE),
        kw.get("ws", FAKE), 1 << 30, None)
    assert call(sel=None) == sa.SA_ERR_INVALID_ARG           # sel and num_sel go together
    assert call(max_sel=0) == sa.SA_ERR_INVALID_ARG
    assert call(out=None) == sa.SA_ERR_INVALID_ARG
    assert call(ws=FAKE + 16) == sa.SA_ERR_INVALID_ARG       # workspace must be 256-byte aligned
    assert call(scale=float("nan")) == sa.SA_ERR_INVALID_ARG


def test_topk_and_meta_argument_checks():
    lib = _lib()
    seqs, cfg = _seqs(), _cfg()
    assert lib.sa_topk_pages(None, 8, ctypes.byref(seqs), ctypes.byref(cfg), FAKE, FAKE, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sa_topk_pages(FAKE, 0, ctypes.byref(seqs), ctypes.byref(cfg), FAKE, FAKE, None) == sa.SA_ERR_INVALID_ARG
    kv = _kv()
    assert lib.sa_build_page_meta(ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(cfg), None, None, None) == sa.SA_ERR_INVALID_ARG
    sals = _cfg(mode=sa.SA_MODE_SALS, unit_tokens=64, proj=FAKE)
    assert lib.sa_build_page_meta(ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(sals), FAKE, None, None) == sa.SA_ERR_INVALID_ARG
    kv3 = _kv(num_kv_heads=3)
    assert lib.sa_build_page_meta(ctypes.byref(kv3), ctypes.byref(seqs), ctypes.byref(sals), FAKE, FAKE, None) == sa.SA_ERR_UNSUPPORTED


def test_append_argument_checks():
    lib = _lib()
    seqs = _seqs()
    sals = _cfg(mode=sa.SA_MODE_SALS, unit_tokens=64, k_compete=32, n_head_forced=0, n_tail_forced=2,
                proj=FAKE)

    def call(kv, cfg, k_new=FAKE, v_new=FAKE, ks=None, vs=None, meta=FAKE, mscale=None):
        return lib.sa_append_kv(k_new, v_new, ks, vs, ctypes.byref(kv), ctypes.byref(seqs),
                                ctypes.byref(cfg), meta, mscale, None)

    assert call(_kv(), _cfg(), k_new=None) == sa.SA_ERR_INVALID_ARG
    assert call(_kv(), _cfg(), v_new=FAKE + 8) == sa.SA_ERR_INVALID_ARG       # 16-byte alignment
    assert call(_kv(), _cfg(), meta=None) == sa.SA_ERR_INVALID_ARG
    i8 = _kv(dtype=sa.SA_I8, k_scale=FAKE, v_scale=FAKE)
    assert call(i8, _cfg(), ks=FAKE, vs=FAKE) == sa.SA_ERR_UNSUPPORTED       # no Quest metadata for int8
    assert call(i8, sals, mscale=FAKE) == sa.SA_ERR_INVALID_ARG              # int8 rows need their scales
    assert call(_kv(), sals) == sa.SA_ERR_INVALID_ARG                        # SALS needs meta_scale
    assert call(_kv(num_kv_heads=3), sals, mscale=FAKE) == sa.SA_ERR_UNSUPPORTED


def test_probe_mode_checks():
    lib = _lib()
    kv, seqs = _kv(), _seqs()
    probe = _cfg(mode=sa.SA_MODE_PROBE, unit_tokens=32, k_compete=6, n_head_forced=0,
                 n_tail_forced=1, n_probe=8)
    assert lib.sa_meta_bytes(ctypes.byref(kv), ctypes.byref(probe)) == 0
    assert lib.sa_meta_scale_bytes(ctypes.byref(kv), ctypes.byref(probe)) == 0
    assert lib.sa_max_units(ctypes.byref(seqs), ctypes.byref(probe)) == 16
    # no metadata to build: success without a launch, even with no buffers
    assert lib.sa_build_page_meta(ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(probe), None, None, None) == sa.SA_OK
    assert _score(lib, kv, seqs, _cfg(mode=sa.SA_MODE_PROBE, unit_tokens=32, n_probe=0)) == sa.SA_ERR_INVALID_ARG
    assert _score(lib, kv, seqs, _cfg(mode=sa.SA_MODE_PROBE, unit_tokens=24, n_probe=8)) == sa.SA_ERR_INVALID_ARG
    assert _score(lib, kv, seqs, probe, scores=None) == sa.SA_ERR_INVALID_ARG


def test_per_head_checks():
    lib = _lib()
    kv, seqs = _kv(), _seqs()
    ph = _cfg(per_head=1)
    assert _score(lib, kv, seqs, _cfg(per_head=2)) == sa.SA_ERR_INVALID_ARG
    sals = _cfg(mode=sa.SA_MODE_SALS, unit_tokens=64, proj=FAKE, per_head=1)
    assert _score(lib, kv, seqs, sals) == sa.SA_ERR_UNSUPPORTED      # per-head selection is Quest's
    assert lib.sa_attn_heads_workspace_size(2, 32, 8, 32, 8) > lib.sa_attn_workspace_size(2, 32, 8, 32, 8)
    assert lib.sa_attn_heads_workspace_size(2, 32, 8, 16385, 8) == 0  # the union supports 16384 pages
    assert lib.sa_attn_heads_workspace_size(2, 32, 8, 32, 0) == 0
    big = _seqs(max_pages=20000)
    need = lib.sa_attn_heads_workspace_size(2, 32, 8, 32, 8)
    call = lambda s, **kw: lib.sa_sparse_decode_attn_heads(
        FAKE, sa.SA_BF16, 32, ctypes.byref(kv), ctypes.byref(s), kw.get("sel", FAKE), kw.get("num", FAKE),
        kw.get("max_sel", 8), 0.088, FAKE, FAKE, kw.get("ws", need), None)
    assert call(seqs, sel=None) == sa.SA_ERR_INVALID_ARG
    assert call(seqs, max_sel=0) == sa.SA_ERR_INVALID_ARG
    assert call(seqs, ws=need - 1) == sa.SA_ERR_WORKSPACE_TOO_SMALL
    assert call(big) == sa.SA_ERR_UNSUPPORTED
    # the step's workspace holds the union attention's (the per-head lists and their partials)
    assert lib.sa_decode_step_workspace_size(32, ctypes.byref(kv), ctypes.byref(seqs), ctypes.byref(ph)) > \
        need


def test_stream_read_argument_checks():
    lib = _lib()
    assert lib.sa_stream_read(None, 1024, ctypes.c_void_p(FAKE), 8, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sa_stream_read(ctypes.c_void_p(FAKE + 4), 1024, ctypes.c_void_p(FAKE), 8, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sa_stream_read(ctypes.c_void_p(FAKE), 1000, ctypes.c_void_p(FAKE), 8, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sa_stream_read(ctypes.c_void_p(FAKE), 0, ctypes.c_void_p(FAKE), 8, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sa_stream_read(ctypes.c_void_p(FAKE), 1024, None, 8, None) == sa.SA_ERR_INVALID_ARG
    assert lib.sa_stream_read(ctypes.c_void_p(FAKE), 1024, ctypes.c_void_p(FAKE), 0, None) == sa.SA_ERR_INVALID_ARG


def test_noalloc_attention_checks():
    """sa_sparse_decode_attn_noalloc validates like sa_sparse_decode_attn and rejects a
    request whose partial records exceed its 32 MiB scratch before any HIP call."""
    lib = _lib()
    kv = sa.sa_kv_cache(FAKE, FAKE, None, None, sa.SA_BF16, 4096, 16, 8, 128)
    big = sa.sa_seqs(FAKE, FAKE, 4096, 16)   # 32768 lists of 16-head groups
    ok = sa.sa_seqs(FAKE, FAKE, 4, 64)
    args = lambda seqs, hq, out: (ctypes.c_void_p(FAKE), sa.SA_BF16, hq, ctypes.byref(kv),  # noqa: E731
                                  ctypes.byref(seqs), ctypes.c_void_p(FAKE), ctypes.c_void_p(FAKE), 16,
                                  0.088, out, None)
    assert lib.sa_sparse_decode_attn_noalloc(*args(big, 128, ctypes.c_void_p(FAKE))) == \
        sa.SA_ERR_WORKSPACE_TOO_SMALL
    assert lib.sa_attn_workspace_size(4096, 128, 8, 16, 16) > 32 << 20
    assert lib.sa_sparse_decode_attn_noalloc(*args(ok, 24, ctypes.c_void_p(FAKE))) == sa.SA_ERR_UNSUPPORTED
    assert lib.sa_sparse_decode_attn_noalloc(*args(ok, 16, None)) == sa.SA_ERR_INVALID_ARG

