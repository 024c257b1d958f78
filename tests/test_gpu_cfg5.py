"""Config 5 at its stated shape against the oracle (run on an MI355X): B=8,
Hq=64, Hkv=8 (group 8), d=128, 262144 tokens per sequence in 16-token pages
(131072 physical pages: K and V hold 2^31 bf16 elements each, so byte offsets
run past 2^32), Quest min/max scoring, a 4096-token budget (254 pages by score
plus the sink and the recent page).

* metadata bit-exact on every page of every sequence;
* every score within the score tolerance (64 lists x 16384 pages);
* the step's selection (benchmark launch configuration and with the page list
  requested) equal to the oracle's up to permitted near-tie swaps, the two
  outputs equal bit for bit, and all 512 query heads within the attention
  tolerance of the oracle evaluated on the GPU's selection;
* the every-page-kept mode ("retention 100% must reproduce full attention",
  SequenceO1 explainer, debugging section): every list keeps all 16384 pages
  and one query head of each of the 64 lists, a different group slot in each,
  equals textbook dense attention over all 262144 tokens.
"""
import os

import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_min_amd as sa
import synth
from sa_testlib import GpuCase, check_attention, check_scores, check_selection, meta_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def cfg5():
    oracle.set_threads(min(16, os.cpu_count() or 1))
    print("[gpu] config 5 full shape: generating inputs", flush=True)
    wl = synth.make_config(5)
    c = GpuCase(wl)
    c.build_meta()
    print(f"[gpu] config 5: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} pages={wl.num_pages} on the GPU",
          flush=True)
    yield wl, c
    oracle.set_threads(1)
    del c
    torch.cuda.empty_cache()


def test_cfg5_metadata_scores_selection_and_step(cfg5):
    wl, c = cfg5
    assert wl.num_pages * 16 * wl.Hkv * wl.d == 1 << 31
    o_meta, _ = oracle.build_meta(wl)
    g_meta, _ = meta_np(c)
    assert np.array_equal(g_meta, o_meta), "metadata differs"
    del g_meta
    print("[gpu] config 5: metadata ok", flush=True)
    g_sc = c.scores().cpu().numpy()
    o_sc, o_ab = oracle.score(wl, o_meta, None)
    check_scores(wl, g_sc, o_sc, o_ab)
    del o_meta, g_sc
    print("[gpu] config 5: scores ok", flush=True)
    out_bench, _, _ = c.step(want_sel=False)
    out_sel, g_sel, g_num = c.step(want_sel=True)
    out_bench, out_sel = out_bench.cpu().numpy(), out_sel.cpu().numpy()
    g_sel, g_num = g_sel.cpu().numpy(), g_num.cpu().numpy()
    assert np.array_equal(out_bench, out_sel), "step output depends on whether the page list is written"
    o_sel, o_num = oracle.select(o_sc, wl.seq_lens, wl.unit_tokens, wl.k_compete, wl.n_head_forced,
                                 wl.n_tail_forced, wl.max_sel)
    swapped = check_selection(wl, g_sel, g_num, o_sel, o_num, o_sc, o_ab)
    assert np.all(g_num == 256)
    # the recent page of the last sequence is the last physical page: its K/V rows end at
    # element 2^31 - 1
    assert np.all(g_sel[7, :, 255] == 16383)
    o_out = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, None, None, wl.page_table,
                             wl.seq_lens, g_sel, g_num, wl.softmax_scale)
    err = check_attention(wl, out_bench, o_out, what="config 5 decode step")
    print(f"[gpu] config 5: step ok (attn err {err:.2e}, swapped lists {len(swapped)})", flush=True)


def test_cfg5_every_page_kept_equals_dense(cfg5):
    wl, c = cfg5
    cfg = sa.SelectCfg(sa.SA_MODE_QUEST, 16, wl.max_units, 1, 1)
    ws = sa.alloc_workspace(sa.sa_decode_step_workspace_size(wl.Hq, c.kv, c.seqs, cfg), c.dev)
    ms = sa.sa_max_selected(c.seqs, cfg)
    assert ms == wl.max_pages
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=c.dev)
    sel = torch.full((wl.B, wl.Hkv, ms), -7, dtype=torch.int32, device=c.dev)
    num = torch.full((wl.B, wl.Hkv), -7, dtype=torch.int32, device=c.dev)
    sa.sa_decode_step(c.d.q, c.kv, c.seqs, cfg, c.meta, None, wl.softmax_scale, out, ws, sel, num)
    num = num.cpu().numpy()
    assert np.all(num == wl.max_pages), "an all-pages budget must keep every page"
    assert np.array_equal(sel.cpu().numpy(), np.broadcast_to(np.arange(wl.max_pages, dtype=np.int32),
                                                             (wl.B, wl.Hkv, wl.max_pages)))
    rows = np.array([b * wl.Hq + h * wl.G + (b + h) % wl.G for b in range(wl.B) for h in range(wl.Hkv)],
                    dtype=np.int32)
    o_out = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, None, None, wl.page_table,
                             wl.seq_lens, None, None, wl.softmax_scale, rows=rows)
    err = check_attention(wl, out.cpu().numpy(), o_out, rows=rows, what="config 5, every page kept")
    print(f"[gpu] config 5 every page kept: ok on {len(rows)} query heads (err {err:.2e})", flush=True)
