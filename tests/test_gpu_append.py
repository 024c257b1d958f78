"""Decode-time append (sa_append_kv) on an MI355X against the oracle's rebuild.

Every case starts from a cache whose last T tokens of each sequence are
missing (their rows zeroed, metadata built for the shorter lengths), then
appends those tokens one decode step at a time.  Afterwards:
  * the K/V cache (and int8 scales) equals the full cache byte for byte;
  * the metadata equals the oracle's build over the final lengths, bit for bit
    (Quest: every referenced page's max/min rows; SALS: every valid token's
    codes and scale) -- the insert-time update folded token by token must
    reach the rebuild exactly ([Quest] page-level min/max maintenance;
    [SALS] per-token index key).
The appended runs cross page starts (slot 0 opens a page) and 64-token block
starts; sequences use a random page table.
"""
import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_min_amd as sa
import synth
from sa_testlib import GpuCase, meta_np

pytestmark = pytest.mark.gpu

T = 40  # appended tokens per sequence

CASES = {
    "quest_f32": dict(B=2, Hq=8, Hkv=8, lens=(300, 529), kv_dtype="f32", q_dtype="f32",
                      mode="quest", budget_pages=8),
    "quest_bf16": dict(B=3, Hq=8, Hkv=2, lens=(57, 256, 1000), kv_dtype="bf16", q_dtype="bf16",
                       mode="quest", budget_pages=8),
    "sals_bf16": dict(B=2, Hq=32, Hkv=8, lens=(300, 700), kv_dtype="bf16", q_dtype="bf16",
                      mode="sals", k_compete=3),
    "sals_i8": dict(B=2, Hq=8, Hkv=2, lens=(129, 640), kv_dtype="i8", q_dtype="bf16", mode="sals",
                    k_compete=3),
    "sals_f32": dict(B=1, Hq=4, Hkv=1, lens=(200,), kv_dtype="f32", q_dtype="f32", mode="sals",
                     k_compete=2),
}


def _rows(wl, lens, b_idx=None):
    """Physical (page, slot) of position lens[b] - 1 for every sequence."""
    t = lens - 1
    pp = wl.page_table[np.arange(wl.B), t // 16]
    return torch.from_numpy(pp.astype(np.int64)), torch.from_numpy((t % 16).astype(np.int64))


@pytest.mark.parametrize("label", sorted(CASES))
def test_append_equals_rebuild(label):
    wl = synth.make_custom(**CASES[label], page_table="random", seed=31, name=label)
    print(f"[gpu] append {label}: B={wl.B} Hkv={wl.Hkv} lens={list(wl.seq_lens)} T={T}", flush=True)
    c = GpuCase(wl)
    d = c.d
    full = {n: getattr(d, n).clone() for n in ("k", "v", "k_scale", "v_scale") if getattr(d, n) is not None}
    L1 = wl.seq_lens.astype(np.int64)
    L0 = L1 - T
    assert L0.min() >= 1
    # remove the last T tokens of every sequence
    for i in range(T):
        pp, sl = _rows(wl, L0 + i + 1)
        for n in full:
            getattr(d, n)[pp.to(c.dev), sl.to(c.dev)] = 0
    d.seq_lens.copy_(torch.from_numpy(L0.astype(np.int32)))
    c.build_meta()
    # append them back, one decode step at a time
    for i in range(T):
        lens_i = L0 + i + 1
        d.seq_lens.copy_(torch.from_numpy(lens_i.astype(np.int32)))
        pp, sl = _rows(wl, lens_i)
        pp, sl = pp.to(c.dev), sl.to(c.dev)
        new = {n: full[n][pp, sl].contiguous() for n in full}
        sa.sa_append_kv(new["k"], new["v"], c.kv, c.seqs, c.cfg, c.meta, c.meta_scale,
                        new.get("k_scale"), new.get("v_scale"))
    torch.cuda.synchronize()
    for n in full:
        assert torch.equal(getattr(d, n), full[n]), f"cache {n} differs after the appends"

    o_meta, o_ms = oracle.build_meta(wl)
    g_meta, g_ms = meta_np(c)
    if wl.mode == "quest":
        for b in range(wl.B):
            for p in range(-(-int(L1[b]) // 16)):
                pp = wl.page_table[b, p]
                assert np.array_equal(g_meta[:, pp].view(np.uint8), o_meta[:, pp].view(np.uint8)), \
                    f"min/max of page (b={b}, p={p}) differs from the rebuild"
    else:
        for b in range(wl.B):
            t = np.arange(L1[b])
            pp, sl = wl.page_table[b, t // 16], t % 16
            assert np.array_equal(g_meta[pp, sl], o_meta[pp, sl]), f"index codes of b={b} differ"
            assert np.array_equal(g_ms[pp, sl], o_ms[pp, sl]), f"index scales of b={b} differ"
    print(f"[gpu] append {label}: ok", flush=True)
