"""Per-head Quest selection on an MI355X against the oracle ([Quest] GQA section:
every query head selects its own pages; the group then reads the union of its
heads' pages once and each head attends over its own pages only).

Per case: per-head scores within the score tolerance, the per-head selection
equal to the oracle's up to permitted near-tie swaps (and bit-exact on the GPU's
own scores), attention over the oracle's per-head lists within the attention
tolerance, and the per-head decode step consistent with both.  Cases cover the
VALU scorer and attention (G = 2, fp32 query), the matrix-core scorer and
attention (G = 4, 8, 16 with bf16), ragged lengths and random page tables.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_min_amd as sa
import synth
from sa_testlib import GpuCase, check_attention, check_scores, check_selection

pytestmark = pytest.mark.gpu

CASES = {
    "ph_gqa2_f32q": dict(B=2, Hq=8, Hkv=4, lens=(1500, 700), kv_dtype="bf16", q_dtype="f32",
                         budget_pages=20, page_table="random"),
    "ph_gqa4_bf16": dict(B=2, Hq=16, Hkv=4, lens=(3000, 1234), kv_dtype="bf16", q_dtype="bf16",
                         budget_pages=32, page_table="random"),
    "ph_gqa8_bf16": dict(B=1, Hq=16, Hkv=2, lens=(4096,), kv_dtype="bf16", q_dtype="bf16",
                         budget_pages=40),
    "ph_gqa16_bf16": dict(B=1, Hq=32, Hkv=2, lens=(2222,), kv_dtype="bf16", q_dtype="bf16",
                          budget_pages=20, page_table="random"),
    "ph_gqa2_f32": dict(B=2, Hq=4, Hkv=2, lens=(900, 1601), kv_dtype="f32", q_dtype="f32",
                        budget_pages=12, page_table="random"),
}


def _union_sizes(sel, num, G):
    B, Hq, _ = sel.shape
    return np.array([[len(set(np.concatenate([sel[b, h * G + g, :num[b, h * G + g]] for g in range(G)])))
                      for h in range(Hq // G)] for b in range(B)])


@pytest.mark.parametrize("label", sorted(CASES))
def test_per_head_step(label):
    _check_per_head(synth.make_custom(**CASES[label], seed=21, name=label), label)


@pytest.mark.parametrize("seed", range(4))
def test_per_head_random(seed):
    r = np.random.default_rng(2000 + seed)
    hkv, G, B = int(r.choice([1, 2, 4])), int(r.choice([2, 4, 8, 16])), int(r.integers(1, 4))
    kw = dict(B=B, Hq=hkv * G, Hkv=hkv, lens=tuple(int(x) for x in r.integers(1, 4001, B)),
              kv_dtype=str(r.choice(["f32", "bf16"])), q_dtype=str(r.choice(["f32", "bf16"])),
              budget_pages=int(r.integers(2, 48)), page_table=str(r.choice(["random", "contiguous"])))
    _check_per_head(synth.make_custom(**kw, seed=600 + seed, name=f"ph_random{seed}"), f"ph_random{seed}: {kw}")


def _check_per_head(wl, label):
    print(f"[gpu] per-head {label}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} lens={list(wl.seq_lens)} "
          f"kv={wl.kv_dtype} q={wl.q_dtype}", flush=True)
    c = GpuCase(wl)
    c.cfg.per_head = 1
    c.build_meta()
    o_meta, _ = oracle.build_meta(wl)
    wl_h = dataclasses.replace(wl, Hkv=wl.Hq)  # one selection list per query head
    # per-head scores
    g_sc_t = torch.full((wl.B, wl.Hq, wl.max_pages), float("nan"), dtype=torch.float32, device=c.dev)
    sa.sa_score_pages(c.q(), c.kv, c.seqs, c.cfg, c.meta, None, g_sc_t)
    g_sc = g_sc_t.cpu().numpy()
    o_sc, o_ab = oracle.quest_scores_per_head(wl.q, wl.q_dtype, o_meta, wl.kv_dtype, wl.page_table,
                                              wl.seq_lens)
    check_scores(wl_h, g_sc, o_sc, o_ab)
    # per-head selection: bit-exact on the GPU's scores, near-tie swaps allowed against the oracle's
    ms = sa.sa_max_selected(c.seqs, c.cfg)
    g_sel_t = torch.full((wl.B, wl.Hq, ms), -7, dtype=torch.int32, device=c.dev)
    g_num_t = torch.full((wl.B, wl.Hq), -7, dtype=torch.int32, device=c.dev)
    sa.sa_topk_pages(g_sc_t, wl.Hq, c.seqs, c.cfg, g_sel_t, g_num_t)
    g_sel, g_num = g_sel_t.cpu().numpy(), g_num_t.cpu().numpy()
    r_sel, r_num = oracle.select(g_sc.astype(np.float64), wl.seq_lens, wl.unit_tokens, wl.k_compete,
                                 wl.n_head_forced, wl.n_tail_forced, wl.max_sel)
    assert np.array_equal(g_sel, r_sel) and np.array_equal(g_num, r_num), "top-K differs on identical scores"
    o_sel, o_num = oracle.select(o_sc, wl.seq_lens, wl.unit_tokens, wl.k_compete, wl.n_head_forced,
                                 wl.n_tail_forced, wl.max_sel)
    swapped = check_selection(wl_h, g_sel, g_num, o_sel, o_num, o_sc, o_ab)
    # attention over the oracle's per-head lists: the group's union read once, each head masked
    o_out = oracle.attention_per_head(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale,
                                      wl.v_scale, wl.page_table, wl.seq_lens, o_sel, o_num,
                                      wl.softmax_scale)
    ws = sa.alloc_workspace(sa.sa_attn_heads_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.max_pages, ms),
                            c.dev)
    g_out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=c.dev)
    sa.sa_sparse_decode_attn_heads(c.q(), c.kv, c.seqs, torch.from_numpy(o_sel).to(c.dev),
                                   torch.from_numpy(o_num).to(c.dev), wl.softmax_scale, g_out, ws)
    err = check_attention(wl, g_out.cpu().numpy(), o_out, what="per-head attention")
    # the per-head decode step: its lists equal the separate top-K's; heads of unswapped
    # lists match the oracle, the others the attention run on the step's own lists
    out, s_sel, s_num = c.step()
    s_sel, s_num = s_sel.cpu().numpy(), s_num.cpu().numpy()
    assert np.array_equal(s_sel, g_sel) and np.array_equal(s_num, g_num), "step selection differs"
    out = out.cpu().numpy().reshape(-1, wl.d)
    rows = np.array([b * wl.Hq + hh for b in range(wl.B) for hh in range(wl.Hq) if (b, hh) not in swapped],
                    dtype=np.int64)
    if len(rows):
        check_attention(wl, out[rows], o_out.reshape(-1, wl.d)[rows], what="per-head step")
    if swapped:
        ref = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=c.dev)
        sa.sa_sparse_decode_attn_heads(c.q(), c.kv, c.seqs, torch.from_numpy(s_sel).to(c.dev),
                                       torch.from_numpy(s_num).to(c.dev), wl.softmax_scale, ref, ws)
        rows2 = np.array([b * wl.Hq + hh for (b, hh) in sorted(swapped)], dtype=np.int64)
        assert np.array_equal(out[rows2], ref.cpu().numpy().reshape(-1, wl.d)[rows2])
    amp = _union_sizes(o_sel, o_num, wl.G) / np.maximum(o_num.reshape(wl.B, wl.Hkv, wl.G).max(-1), 1)
    print(f"[gpu] per-head {label}: ok (attn err {err:.2e}, swapped {len(swapped)}, "
          f"union / list length {amp.mean():.2f})", flush=True)
