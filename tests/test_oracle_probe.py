"""Pins of the oracle's probe-sampling scorer ([RK] §1-§2: a block's score is the
largest query-key dot product over keys probed evenly inside the block).

  * the probed positions follow the page's rule, step = max(1, len / n_probe):
    a 32-token block with 8 probes reads positions 0, 4, ..., 28 of the block,
    a shorter last block reads every position; a needle is seen exactly when
    it sits on a probed position;
  * with n_probe >= block length every key is probed and the score is the
    block's exact largest logit, checked against a dense matmul and max;
  * GQA groups take the max over their query heads; int8 keys are code x scale.
"""
import numpy as np
import pytest

import oracle

D = 128


def _case(L, U, n_probe, hq=1, hkv=1, kv_dtype="f32", seed=0, k=None, q=None):
    rng = np.random.default_rng(seed)
    n_pages = -(-L // 16)
    if k is None:
        k = rng.standard_normal((n_pages, 16, hkv, D)).astype(np.float32)
    if q is None:
        q = rng.standard_normal((1, hq, D)).astype(np.float32)
    pt = rng.permutation(n_pages).astype(np.int32)[None, :]
    ks = None
    if kv_dtype == "i8":
        ks = (rng.uniform(0.01, 0.05, (n_pages, 16, hkv)).astype(np.float16)).view(np.uint16)
        k = rng.integers(-127, 128, (n_pages, 16, hkv, D)).astype(np.int8)
    sc, ab = oracle.probe_scores(q, "f32", k, kv_dtype, ks, pt, np.array([L], np.int32), U, n_probe)
    return sc, ab, k, q, pt, ks


def _keys(k, pt, hkv_h, positions, ks=None):
    """Dense [len(positions), D] keys of kv-head hkv_h at logical positions."""
    rows = []
    for t in positions:
        pp, s = pt[0, t // 16], t % 16
        row = k[pp, s, hkv_h].astype(np.float64)
        if ks is not None:
            row = row * float(ks[pp, s, hkv_h].view(np.float16))
        rows.append(row)
    return np.array(rows)


def test_probe_positions_follow_the_rule():
    L, U = 40, 32  # block 0: 32 tokens (step 4); block 1: 8 tokens (step 1)
    base = np.zeros((3, 16, 1, D), np.float32)
    q = np.ones((1, 1, D), np.float32)
    rng = np.random.default_rng(3)
    pt = rng.permutation(3).astype(np.int32)[None, :]
    for t, seen in [(0, True), (4, True), (28, True), (5, False), (31, False), (3, False),
                    (33, True), (39, True)]:
        k = base.copy()
        k[pt[0, t // 16], t % 16, 0, :] = 1.0  # needle: q . k = 128 at position t only
        sc, _ = oracle.probe_scores(q, "f32", k, "f32", None, pt, np.array([L], np.int32), U, 8)
        u = t // U
        assert sc[0, 0, u] == (128.0 if seen else 0.0), (t, sc[0, 0, u])
        assert sc[0, 0, 1 - u] == 0.0


@pytest.mark.parametrize("L,U", [(64, 32), (50, 16), (45, 64)])
def test_all_probed_equals_exact_max_logit(L, U):
    sc, ab, k, q, pt, _ = _case(L, U, n_probe=U, seed=L)
    for u in range(-(-L // U)):
        pos = list(range(u * U, min((u + 1) * U, L)))
        logits = _keys(k, pt, 0, pos) @ q[0, 0].astype(np.float64)
        assert sc[0, 0, u] == pytest.approx(logits.max(), rel=1e-12, abs=1e-12)
    assert np.all(np.isneginf(sc[0, 0, -(-L // U):]))


def test_group_max_and_int8_keys():
    L, U, npb = 96, 32, 8
    sc, ab, k, q, pt, ks = _case(L, U, npb, hq=4, hkv=2, kv_dtype="i8", seed=11)
    for h in range(2):
        for u in range(L // U):
            pos = list(range(u * U, (u + 1) * U, U // npb))
            kk = _keys(k, pt, h, pos, ks)
            logits = kk @ q[0, 2 * h:2 * h + 2].astype(np.float64).T  # the group's two heads
            assert sc[0, h, u] == pytest.approx(logits.max(), rel=1e-12)
            assert ab[0, h, u] == pytest.approx(np.abs(kk[:, None, :] * q[0, 2 * h:2 * h + 2][None]).sum(-1).max(), rel=1e-12)
