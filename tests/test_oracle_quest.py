"""Pins of the oracle's Quest metadata and page scorer.

Each check comes from the mathematics the pages state (Quest explainer:
min/max metadata, upper-bound inequality and its case proof, incremental
update; GQA section) and is computed independently of the oracle's C code.
"""
import numpy as np
import pytest

import oracle
import synth


def _kv_f64(wl, x):
    return synth.bf16_to_f32(x).astype(np.float64) if wl.kv_dtype == "bf16" else x.astype(np.float64)


def _q_f64(wl, q=None):
    q = wl.q if q is None else q
    return synth.bf16_to_f32(q).astype(np.float64) if wl.q_dtype == "bf16" else q.astype(np.float64)


def _tokens(wl, b, p):
    """(physical page, number of valid slots) of logical page p of sequence b."""
    L = int(wl.seq_lens[b])
    return int(wl.page_table[b, p]), min(16, L - 16 * p)


CASES = [
    dict(B=2, Hq=4, Hkv=4, lens=(100, 37), kv_dtype="f32", q_dtype="f32", page_table="random"),
    dict(B=3, Hq=8, Hkv=2, lens=(257, 16, 1), kv_dtype="bf16", q_dtype="bf16", page_table="random"),
    dict(B=1, Hq=8, Hkv=1, lens=(64,), kv_dtype="bf16", q_dtype="bf16"),
]


@pytest.mark.parametrize("case", CASES)
def test_meta_is_bruteforce_min_max(case):
    wl = synth.make_custom(**case, seed=21)
    meta = oracle.quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens)
    K = _kv_f64(wl, wl.k)
    M = _kv_f64(wl, meta)
    for b in range(wl.B):
        for p in range(wl.n_pages(b)):
            pp, nv = _tokens(wl, b, p)
            keys = K[pp, :nv]  # [nv, Hkv, d]
            assert np.array_equal(M[:, pp, 0], keys.max(axis=0))
            assert np.array_equal(M[:, pp, 1], keys.min(axis=0))
            # every bound value is attained by a valid token of the page
            assert np.all((keys == M[:, pp, 0][None]).any(axis=0))
            assert np.all((keys == M[:, pp, 1][None]).any(axis=0))


def test_meta_matches_incremental_update():
    """Folding M <- max(M, k), m <- min(m, k) token by token (the insert-time update)
    gives the same metadata as the oracle's whole-page build."""
    wl = synth.make_custom(B=1, Hq=2, Hkv=2, lens=(45,), kv_dtype="bf16", seed=5)
    meta = oracle.quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens)
    K = _kv_f64(wl, wl.k)
    for p in range(wl.n_pages(0)):
        pp, nv = _tokens(wl, 0, p)
        Mx = np.full(K.shape[2:], -np.inf)
        mn = np.full(K.shape[2:], np.inf)
        for s in range(nv):
            Mx = np.maximum(Mx, K[pp, s])
            mn = np.minimum(mn, K[pp, s])
        assert np.array_equal(_kv_f64(wl, meta[:, pp, 0]), Mx)
        assert np.array_equal(_kv_f64(wl, meta[:, pp, 1]), mn)


@pytest.mark.parametrize("case", CASES)
def test_bound_dominates_every_true_dot(case):
    wl = synth.make_custom(**case, seed=22)
    meta = oracle.quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens)
    sc, ab = oracle.quest_scores(wl.q, wl.q_dtype, meta, wl.kv_dtype, wl.page_table, wl.seq_lens)
    K = _kv_f64(wl, wl.k)
    Q = _q_f64(wl)
    G = wl.G
    for b in range(wl.B):
        for h in range(wl.Hkv):
            for p in range(wl.max_pages):
                if p >= wl.n_pages(b):
                    assert sc[b, h, p] == -np.inf
                    continue
                pp, nv = _tokens(wl, b, p)
                dots = Q[b, h * G:(h + 1) * G] @ K[pp, :nv, h].T  # [G, nv]
                assert sc[b, h, p] >= dots.max() - 1e-12 * ab[b, h, p]
                assert ab[b, h, p] >= abs(sc[b, h, p]) - 1e-12 * ab[b, h, p]


@pytest.mark.parametrize("case", CASES)
def test_bound_equals_linear_form(case):
    """sum_i max(q_i m_i, q_i M_i) = q+ . M + q- . m (the two sign cases of the proof)."""
    wl = synth.make_custom(**case, seed=23)
    meta = oracle.quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens)
    sc, ab = oracle.quest_scores(wl.q, wl.q_dtype, meta, wl.kv_dtype, wl.page_table, wl.seq_lens)
    Mt = _kv_f64(wl, meta)
    Q = _q_f64(wl)
    G = wl.G
    for b in range(wl.B):
        for p in range(wl.n_pages(b)):
            pp = int(wl.page_table[b, p])
            for h in range(wl.Hkv):
                qg = Q[b, h * G:(h + 1) * G]
                lin = np.maximum(qg, 0) @ Mt[h, pp, 0] + np.minimum(qg, 0) @ Mt[h, pp, 1]
                assert abs(sc[b, h, p] - lin.max()) <= 1e-12 * ab[b, h, p]


def test_one_hot_query_reads_one_bound():
    """q = +e_i scores M_i, q = -e_i scores -m_i (catches swapped or mis-indexed slots)."""
    wl = synth.make_custom(B=1, Hq=2, Hkv=2, lens=(80,), kv_dtype="f32", q_dtype="f32", seed=9)
    meta = oracle.quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens)
    for i in (0, 17, 127):
        for sign in (1.0, -1.0):
            q = np.zeros_like(wl.q)
            q[0, :, i] = sign
            sc, _ = oracle.quest_scores(q, "f32", meta, "f32", wl.page_table, wl.seq_lens)
            for p in range(wl.n_pages(0)):
                pp = int(wl.page_table[0, p])
                for h in range(2):
                    want = meta[h, pp, 0, i] if sign > 0 else -meta[h, pp, 1, i]
                    assert sc[0, h, p] == want


def test_bound_is_positively_homogeneous():
    wl = synth.make_custom(B=2, Hq=8, Hkv=4, lens=(200, 33), kv_dtype="bf16", q_dtype="f32", seed=4)
    meta = oracle.quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens)
    s1, _ = oracle.quest_scores(wl.q, "f32", meta, "bf16", wl.page_table, wl.seq_lens)
    for c in (2.0, 0.25, 8.0):
        s2, _ = oracle.quest_scores((wl.q * c).astype(np.float32), "f32", meta, "bf16",
                                    wl.page_table, wl.seq_lens)
        fin = np.isfinite(s1)
        assert np.array_equal(s2[fin], c * s1[fin])


def test_identical_keys_make_the_bound_exact():
    """A page whose keys are all equal has m = M = k, so the bound is q.k itself."""
    wl = synth.make_custom(B=1, Hq=1, Hkv=1, lens=(64,), kv_dtype="f32", q_dtype="f32", seed=8)
    wl.k[:, :, :, :] = wl.k[:, :1, :, :]
    meta = oracle.quest_meta(wl.k, "f32", wl.page_table, wl.seq_lens)
    sc, ab = oracle.quest_scores(wl.q, "f32", meta, "f32", wl.page_table, wl.seq_lens)
    for p in range(4):
        dot = wl.q[0, 0].astype(np.float64) @ wl.k[p, 0, 0].astype(np.float64)
        assert abs(sc[0, 0, p] - dot) <= 1e-12 * ab[0, 0, p]


def test_group_score_is_max_over_heads():
    """With G heads sharing a kv-head, the group score is the max of the G single-head scores."""
    wl = synth.make_custom(B=1, Hq=8, Hkv=2, lens=(96,), kv_dtype="bf16", q_dtype="bf16", seed=12)
    meta = oracle.quest_meta(wl.k, "bf16", wl.page_table, wl.seq_lens)
    sc, _ = oracle.quest_scores(wl.q, "bf16", meta, "bf16", wl.page_table, wl.seq_lens)
    for g in range(4):
        qh = np.ascontiguousarray(wl.q[:, g::4])  # heads g and 4+g -> kv-heads 0 and 1
        s1, _ = oracle.quest_scores(qh, "bf16", meta, "bf16", wl.page_table, wl.seq_lens)
        assert np.all(s1 <= sc)
    per_head = np.stack([oracle.quest_scores(np.ascontiguousarray(wl.q[:, g::4]), "bf16", meta, "bf16",
                                             wl.page_table, wl.seq_lens)[0] for g in range(4)])
    assert np.array_equal(per_head.max(axis=0), sc)


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_strong_needle_is_always_selected(kv_dtype):
    """Needle theorem: if alpha*|q| exceeds every other middle page's score, the needle
    page's bound (>= its true dot alpha*|q|) is the largest, so any k >= 1 keeps it."""
    for seed in range(6):
        wl = synth.make_custom(B=1, Hq=4, Hkv=4, lens=(16 * 40 - 3,), kv_dtype=kv_dtype,
                               q_dtype=kv_dtype, budget_pages=3, seed=100 + seed)
        meta = oracle.quest_meta(wl.k, kv_dtype, wl.page_table, wl.seq_lens)
        sc, _ = oracle.quest_scores(wl.q, kv_dtype, meta, kv_dtype, wl.page_table, wl.seq_lens)
        n = wl.n_pages(0)
        Q = _q_f64(wl)
        needle_pages = synth.uniform_int(seed, 77, wl.Hkv, 1, n - 2)
        for h in range(wl.Hkv):
            p = int(needle_pages[h])
            others = np.delete(sc[0, h, 1:n - 1], p - 1)
            qn = np.linalg.norm(Q[0, h])
            alpha = 1.25 * max(others.max(), 1e-3) / qn
            key = (alpha * Q[0, h] / qn).astype(np.float32)
            slot = (seed * 5 + h) % 16
            wl.k[p, slot, h] = key if kv_dtype == "f32" else synth.f32_to_bf16(key)
        meta = oracle.quest_meta(wl.k, kv_dtype, wl.page_table, wl.seq_lens)
        _, sel, num, sc2, _ = oracle.decode_step(wl, meta, None)
        for h in range(wl.Hkv):
            p = int(needle_pages[h])
            assert p in sel[0, h, :num[0, h]]
            assert np.argmax(sc2[0, h, 1:n - 1]) + 1 == p
