"""Pins of the oracle's attention over selected pages.

Retention of every page must reproduce full attention (SequenceO1 explainer,
debugging section), which is the textbook softmax(q K^T / sqrt(d)) V; the
int8 path dequantises code * per-token scale (SALS on Ascend, SFAA; Day 10·2,
exact attention on the selected set).  The textbook reference here is torch's
CPU scaled_dot_product_attention in float64, an independent implementation.
"""
import numpy as np
import pytest
import torch

import oracle
import synth


def _f64(x, dtype, scale=None):
    if dtype == "bf16":
        return synth.bf16_to_f32(x).astype(np.float64)
    if dtype == "i8":
        return x.astype(np.float64) * synth.f16_to_f32(scale).astype(np.float64)[..., None]
    return x.astype(np.float64)


def _dense_torch(wl, q=None):
    """Textbook attention per (b, head) over positions [0, L_b) via torch SDPA in float64."""
    q = wl.q if q is None else q
    Q = _f64(q, wl.q_dtype)
    K = _f64(wl.k, wl.kv_dtype, wl.k_scale)
    V = _f64(wl.v, wl.kv_dtype, wl.v_scale)
    out = np.zeros((wl.B, wl.Hq, wl.d))
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        pages = wl.page_table[b, :wl.n_pages(b)]
        kb = K[pages].reshape(-1, wl.Hkv, wl.d)[:L]  # [L, Hkv, d] in logical order
        vb = V[pages].reshape(-1, wl.Hkv, wl.d)[:L]
        for hq in range(wl.Hq):
            h = hq // wl.G
            o = torch.nn.functional.scaled_dot_product_attention(
                torch.from_numpy(Q[b, hq][None, None, None]),
                torch.from_numpy(np.ascontiguousarray(kb[:, h])[None, None]),
                torch.from_numpy(np.ascontiguousarray(vb[:, h])[None, None]),
                scale=wl.softmax_scale)
            out[b, hq] = o.numpy().reshape(-1)
    return out


CASES = [
    dict(B=2, Hq=4, Hkv=4, lens=(100, 37), kv_dtype="f32", q_dtype="f32", page_table="random"),
    dict(B=3, Hq=8, Hkv=2, lens=(257, 16, 1), kv_dtype="bf16", q_dtype="bf16", page_table="random"),
    dict(B=2, Hq=8, Hkv=2, lens=(300, 129), kv_dtype="i8", q_dtype="bf16", page_table="random"),
]


@pytest.mark.parametrize("case", CASES)
def test_dense_attention_is_textbook_softmax(case):
    wl = synth.make_custom(**case, seed=31)
    out = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale,
                           wl.page_table, wl.seq_lens, None, None, wl.softmax_scale)
    ref = _dense_torch(wl)
    assert np.allclose(out, ref, rtol=2e-7, atol=2e-7)


@pytest.mark.parametrize("case", CASES)
def test_all_pages_selected_equals_dense(case):
    """Budget >= every unit: the decode step's output equals dense attention."""
    wl = synth.make_custom(**case, seed=32, budget_pages=10 ** 4)
    if wl.kv_dtype == "i8":
        pytest.skip("Quest metadata is built on f32/bf16 caches")
    meta, ms = oracle.build_meta(wl)
    out, sel, num, _, _ = oracle.decode_step(wl, meta, ms)
    for b in range(wl.B):
        assert np.all(num[b] == wl.n_pages(b))
    dense = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale,
                             wl.page_table, wl.seq_lens, None, None, wl.softmax_scale)
    assert np.array_equal(out, dense)


def test_single_token_returns_its_value():
    wl = synth.make_custom(B=2, Hq=4, Hkv=2, lens=(1, 1), kv_dtype="f32", q_dtype="f32", seed=3)
    out = oracle.attention(wl.q, "f32", wl.k, wl.v, "f32", None, None, wl.page_table, wl.seq_lens,
                           None, None, wl.softmax_scale)
    for b in range(2):
        pp = wl.page_table[b, 0]
        for hq in range(4):
            assert np.array_equal(out[b, hq], wl.v[pp, 0, hq // 2])


def test_zero_query_gives_mean_of_selected_values():
    wl = synth.make_custom(B=1, Hq=2, Hkv=2, lens=(16 * 9 + 5,), kv_dtype="bf16", q_dtype="bf16",
                           page_table="random", seed=4)
    q0 = np.zeros_like(wl.q)
    sel = np.full((1, 2, 4), -1, dtype=np.int32)
    sel[0, 0, :3] = [0, 4, 9]
    sel[0, 1, :4] = [1, 2, 3, 9]
    num = np.array([[3, 4]], dtype=np.int32)
    out = oracle.attention(q0, "bf16", wl.k, wl.v, "bf16", None, None, wl.page_table, wl.seq_lens,
                           sel, num, wl.softmax_scale)
    V = _f64(wl.v, "bf16")
    for h in range(2):
        rows = []
        for p in sel[0, h, :num[0, h]]:
            nv = min(16, int(wl.seq_lens[0]) - 16 * int(p))
            rows.append(V[wl.page_table[0, p], :nv, h])
        want = np.concatenate(rows).mean(axis=0)
        assert np.allclose(out[0, h], want, rtol=1e-6, atol=1e-7)


def test_physical_page_permutation_invariance():
    wl = synth.make_custom(B=2, Hq=4, Hkv=2, lens=(200, 77), kv_dtype="bf16", q_dtype="bf16", seed=5)
    out1 = oracle.attention(wl.q, "bf16", wl.k, wl.v, "bf16", None, None, wl.page_table,
                            wl.seq_lens, None, None, wl.softmax_scale)
    perm = synth.permutation(9, 9, wl.num_pages)
    inv = np.argsort(perm)
    k2, v2 = np.empty_like(wl.k), np.empty_like(wl.v)
    k2[perm] = wl.k
    v2[perm] = wl.v
    pt2 = np.where(wl.page_table >= 0, perm[np.maximum(wl.page_table, 0)], -1).astype(np.int32)
    out2 = oracle.attention(wl.q, "bf16", k2, v2, "bf16", None, None, pt2, wl.seq_lens, None, None,
                            wl.softmax_scale)
    assert np.array_equal(out1, out2)
    assert np.array_equal(inv[perm], np.arange(wl.num_pages))


def test_int8_path_equals_float_path_on_dequantised_values():
    wl = synth.make_custom(B=1, Hq=4, Hkv=2, lens=(150,), kv_dtype="i8", q_dtype="bf16", seed=6)
    kf = (wl.k.astype(np.float32) * synth.f16_to_f32(wl.k_scale)[..., None]).astype(np.float32)
    vf = (wl.v.astype(np.float32) * synth.f16_to_f32(wl.v_scale)[..., None]).astype(np.float32)
    a = oracle.attention(wl.q, "bf16", wl.k, wl.v, "i8", wl.k_scale, wl.v_scale, wl.page_table,
                         wl.seq_lens, None, None, wl.softmax_scale)
    b = oracle.attention(wl.q, "bf16", kf, vf, "f32", None, None, wl.page_table, wl.seq_lens, None,
                         None, wl.softmax_scale)
    assert np.array_equal(a, b)


def test_row_subset_matches_full_output():
    wl = synth.make_custom(B=2, Hq=8, Hkv=2, lens=(90, 33), kv_dtype="bf16", q_dtype="bf16", seed=7)
    full = oracle.attention(wl.q, "bf16", wl.k, wl.v, "bf16", None, None, wl.page_table,
                            wl.seq_lens, None, None, wl.softmax_scale)
    rows = np.array([0, 5, 9, 15], dtype=np.int32)
    sub = oracle.attention(wl.q, "bf16", wl.k, wl.v, "bf16", None, None, wl.page_table,
                           wl.seq_lens, None, None, wl.softmax_scale, rows=rows)
    assert np.array_equal(sub, full.reshape(-1, wl.d)[rows])


def test_masked_tail_tokens_are_ignored():
    """Garbage in slots past the sequence end must not change the output."""
    wl = synth.make_custom(B=1, Hq=2, Hkv=2, lens=(37,), kv_dtype="f32", q_dtype="f32", seed=8)
    out1 = oracle.attention(wl.q, "f32", wl.k, wl.v, "f32", None, None, wl.page_table, wl.seq_lens,
                            None, None, wl.softmax_scale)
    wl.k[wl.page_table[0, 2], 5:] = 1e3
    wl.v[wl.page_table[0, 2], 5:] = -1e3
    out2 = oracle.attention(wl.q, "f32", wl.k, wl.v, "f32", None, None, wl.page_table, wl.seq_lens,
                            None, None, wl.softmax_scale)
    assert np.array_equal(out1, out2)
