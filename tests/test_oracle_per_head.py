"""Pins of the oracle's per-head selection ([Quest] GQA section: each query head
selects its own pages instead of one selection per group).

  * with one query head per group, per-head scores are the group scores;
  * a group of identical heads gives every head the group score;
  * head h*G + g's score is the group score of a query whose whole group is
    replaced by head g's vector (a wrong head-to-row mapping fails this);
  * per-head attention with every head given every page is dense attention,
    and changing one head's page list changes that head's output only.
"""
import numpy as np

import oracle
import synth


def _wl(Hq, Hkv, seed=3):
    return synth.make_custom(B=2, Hq=Hq, Hkv=Hkv, lens=(700, 333), kv_dtype="bf16", q_dtype="f32",
                             budget_pages=8, page_table="random", seed=seed)


def _group(wl, q):
    meta = oracle.quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens)
    return oracle.quest_scores(q, "f32", meta, wl.kv_dtype, wl.page_table, wl.seq_lens), meta


def test_one_head_per_group_equals_group_scores():
    wl = _wl(4, 4)
    (sc, ab), meta = _group(wl, wl.q)
    ph, pa = oracle.quest_scores_per_head(wl.q, "f32", meta, wl.kv_dtype, wl.page_table, wl.seq_lens)
    assert np.array_equal(ph, sc) and np.array_equal(pa, ab)


def test_identical_heads_take_the_group_score():
    wl = _wl(8, 2)
    q = np.repeat(wl.q[:, ::4], 4, axis=1)  # every head of a group equals its first head
    (sc, _), meta = _group(wl, q)
    ph, _ = oracle.quest_scores_per_head(q, "f32", meta, wl.kv_dtype, wl.page_table, wl.seq_lens)
    for g in range(4):
        assert np.array_equal(ph[:, g::4], sc)


def test_head_rows_map_to_their_own_query():
    wl = _wl(8, 2)
    meta = oracle.quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens)
    ph, _ = oracle.quest_scores_per_head(wl.q, "f32", meta, wl.kv_dtype, wl.page_table, wl.seq_lens)
    for g in range(4):
        qg = np.repeat(wl.q[:, g::4], 4, axis=1)  # group h made of copies of head h*4 + g
        sc, _ = oracle.quest_scores(qg, "f32", meta, wl.kv_dtype, wl.page_table, wl.seq_lens)
        assert np.array_equal(ph[:, g::4], sc), g


def test_per_head_attention_reduces_to_dense_and_is_head_local():
    wl = _wl(8, 2)
    n = np.array([wl.n_pages(b) for b in range(wl.B)])
    mp = wl.max_pages
    sel = np.full((wl.B, wl.Hq, mp), -1, np.int32)
    for b in range(wl.B):
        sel[b, :, :n[b]] = np.arange(n[b])
    num = np.repeat(n[:, None], wl.Hq, axis=1).astype(np.int32)
    args = (wl.q, "f32", wl.k, wl.v, wl.kv_dtype, None, None, wl.page_table, wl.seq_lens)
    full = oracle.attention_per_head(*args, sel, num, wl.softmax_scale)
    dense = oracle.attention(*args, None, None, wl.softmax_scale)
    assert np.array_equal(full, dense)
    sel2, num2 = sel.copy(), num.copy()
    sel2[1, 5, :] = -1
    sel2[1, 5, :3] = [0, 2, 4]
    num2[1, 5] = 3
    part = oracle.attention_per_head(*args, sel2, num2, wl.softmax_scale)
    changed = np.argwhere(np.any(part != full, axis=-1))
    assert changed.tolist() == [[1, 5]]
