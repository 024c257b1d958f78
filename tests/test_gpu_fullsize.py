"""GPU-vs-oracle parity at the workloads' full sizes, with the decode step run in
the launch configuration the benchmark times (no page list requested), plus the
same step with the page list requested (run on an MI355X).

Every config is checked end to end:
  * metadata / index key bit-exact on every page of every sequence;
  * scores within the score tolerance on every unit;
  * the step's selection equal to the oracle's up to permitted near-tie swaps;
  * the step's output (benchmark configuration) equal, bit for bit, to the output of
    the same step with the page list requested, and within the attention tolerance
    of the oracle evaluated on the GPU's selected pages, for every query head.

Configs: 1 (fp32 MHA, 2K), 2 (bf16 MHA, 32K: the benchmark workload), 3 (GQA-4,
ragged 8K-32K, random page table), 4 (SALS, int8 KV, 128K), and config 5 as one
GPU's kv-head share (B=8, Hq=8, Hkv=1, 256K), also with an all-pages budget
against dense attention.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from sa_testlib import GpuCase, check_attention, check_scores, check_selection, meta_np

pytestmark = pytest.mark.gpu


def _cfg5_share(dense=False):
    wl = synth.make_custom(B=8, Hq=8, Hkv=1, lens=(262144,) * 8, kv_dtype="bf16", q_dtype="bf16",
                           budget_pages=4096 // 16, seed=5000, name="cfg5-share")
    if dense:
        wl.k_compete = wl.max_units
        wl.name += "-dense"
    return wl


def _workload(name):
    if name == "cfg5-share":
        return _cfg5_share()
    if name == "cfg5-share-dense":
        return _cfg5_share(dense=True)
    return synth.make_config(int(name[3:]))


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "cfg3", "cfg4", "cfg5-share"])
def test_full_size_step(name):
    wl = _workload(name)
    print(f"[gpu] full-size {name}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} max_pages={wl.max_pages} "
          f"kv={wl.kv_dtype} mode={wl.mode}", flush=True)
    c = GpuCase(wl)
    c.build_meta()
    o_meta, o_ms = oracle.build_meta(wl)
    g_meta, g_ms = meta_np(c)
    if wl.mode == "quest":
        assert np.array_equal(g_meta.view(np.uint8), o_meta.view(np.uint8)), "metadata differs"
    else:
        assert np.array_equal(g_meta, o_meta), "index codes differ"
        assert np.array_equal(g_ms, o_ms), "index scales differ"
    g_sc = c.scores().cpu().numpy()
    o_sc, o_ab = oracle.score(wl, o_meta, o_ms)
    check_scores(wl, g_sc, o_sc, o_ab)
    print(f"[gpu] full-size {name}: metadata and scores ok", flush=True)

    out_bench, _, _ = c.step(want_sel=False)  # the benchmark's launch configuration
    out_sel, g_sel, g_num = c.step(want_sel=True)
    out_bench, out_sel = out_bench.cpu().numpy(), out_sel.cpu().numpy()
    g_sel, g_num = g_sel.cpu().numpy(), g_num.cpu().numpy()
    assert np.array_equal(out_bench, out_sel), "step output depends on whether the page list is written"
    o_sel, o_num = oracle.select(o_sc, wl.seq_lens, wl.unit_tokens, wl.k_compete, wl.n_head_forced,
                                 wl.n_tail_forced, wl.max_sel)
    swapped = check_selection(wl, g_sel, g_num, o_sel, o_num, o_sc, o_ab)
    o_out = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale,
                             wl.page_table, wl.seq_lens, g_sel, g_num, wl.softmax_scale)
    err = check_attention(wl, out_bench, o_out, what=f"{name} decode step")
    print(f"[gpu] full-size {name}: ok (attn err {err:.2e}, swapped lists {len(swapped)})", flush=True)


def test_full_size_all_pages_equals_dense():
    """Config 5's share with a budget of every page: the step keeps all pages and
    equals textbook dense attention (sampled query heads, every token)."""
    wl = _workload("cfg5-share-dense")
    print(f"[gpu] full-size {wl.name}: dense equivalence", flush=True)
    c = GpuCase(wl)
    c.build_meta()
    out, sel, num = c.step(want_sel=True)
    num = num.cpu().numpy()
    assert np.all(num == wl.max_pages), "an all-pages budget must keep every page"
    rows = np.array([0, 9, 18, 27, 36, 45, 54, 63], dtype=np.int32)  # one head of each sequence
    sel_all = np.tile(np.arange(wl.max_pages, dtype=np.int32), (wl.B, wl.Hkv, 1))
    o_out = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale,
                             wl.page_table, wl.seq_lens, sel_all, num, wl.softmax_scale, rows=rows)
    err = check_attention(wl, out.cpu().numpy(), o_out, rows=rows, what="dense-equivalent step")
    print(f"[gpu] full-size {wl.name}: ok (attn err {err:.2e})", flush=True)
