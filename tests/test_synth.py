"""Generator determinism, distributions, conversions and the bytes model."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import synth

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def test_normal_deterministic_and_piecewise():
    a = synth.normal(11, 2, (1000,))
    b = synth.normal(11, 2, (1000,))
    assert np.array_equal(a, b)
    c = np.concatenate([synth.normal(11, 2, (337,)), synth.normal(11, 2, (663,), offset=337)])
    assert np.array_equal(a, c)
    assert not np.array_equal(a, synth.normal(12, 2, (1000,)))
    assert not np.array_equal(a, synth.normal(11, 3, (1000,)))


def test_normal_thread_count_independent():
    code = ("import sys; sys.path.insert(0, %r); import synth, hashlib; "
            "print(hashlib.sha1(synth.normal(5, 9, (200001,), 'bf16').tobytes()).hexdigest())"
            % os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    outs = set()
    for t in ("1", "3"):
        env = dict(os.environ, OMP_NUM_THREADS=t)
        outs.add(subprocess.check_output([sys.executable, "-c", code], env=env).strip())
    assert len(outs) == 1


def test_normal_moments():
    x = synth.normal(3, 1, (1 << 20,)).astype(np.float64)
    assert abs(x.mean()) < 5e-3
    assert abs(x.std() - 1.0) < 5e-3
    # Box-Muller tails: P(|z| > 3) = 0.0027
    assert abs((np.abs(x) > 3).mean() - 0.0027) < 4e-4


def test_bf16_rounding_matches_definition():
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa (1.0) wins
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -2.5, 3.1415926], dtype=np.float32)
    bits = synth.f32_to_bf16(vals)
    assert bits[0] == 0x3F80 and bits[1] == 0x3F80 and bits[2] == 0x3F82
    back = synth.bf16_to_f32(bits)
    assert back[3] == -2.5
    assert abs(back[4] - np.float32(3.1415926)) <= 2 ** -7 * 2


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.uniform(-9, 4.8, 20000),
                        [0.0, -0.0, 65504.0, 65519.0, 65520.0, 2 ** -24, 2 ** -25, 3 * 2 ** -26,
                         6.1e-5, 1e-7]]).astype(np.float32)
    ours = synth.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.f16_to_f32(ref), ref.view(np.float16).astype(np.float32))


def test_int8_quantisation_format():
    x = synth.normal(4, 2, (300, 128))
    codes, sc = synth.quant_int8_rows(x)
    s = synth.f16_to_f32(sc)
    assert codes.min() >= -127 and codes.max() <= 127
    assert np.all(np.abs(codes).max(axis=1) >= 126)
    err = np.abs(x - codes.astype(np.float32) * s[:, None])
    assert np.all(err <= s[:, None] * 0.5 * (1 + 1e-6) + 1e-30)
    z, zs = synth.quant_int8_rows(np.zeros((2, 128), np.float32))
    assert not z.any() and not zs.any()


def test_uniform_int_and_permutation():
    u = synth.uniform_int(1, 1, 100000, 3, 9)
    assert u.min() == 3 and u.max() == 9
    p = synth.permutation(2, 3, 1000)
    assert np.array_equal(np.sort(p), np.arange(1000))
    assert not np.array_equal(p, np.arange(1000))


def test_workload_shapes_and_needles():
    wl = synth.make_config(1)
    assert wl.k.shape == (128, 16, 8, 128) and wl.k.dtype == np.float32
    assert wl.k_compete == 14 and wl.max_sel == 16
    assert len(wl.needles) == 8
    for b, h, p, s in wl.needles:
        assert 1 <= p <= 126
        key = wl.k[wl.page_table[b, p], s, h].astype(np.float64)
        qh = wl.q[b, h].astype(np.float64)
        assert np.allclose(key, 4 * qh / np.linalg.norm(qh), atol=1e-6)


def test_random_page_table_is_a_partition():
    wl = synth.make_custom(B=5, Hq=4, Hkv=2, lens=(17, 300, 1, 64, 129), page_table="random", seed=3)
    used = np.concatenate([wl.page_table[b, :wl.n_pages(b)] for b in range(5)])
    assert np.array_equal(np.sort(used), np.arange(wl.num_pages))
    for b in range(5):
        assert np.all(wl.page_table[b, wl.n_pages(b):] == -1)


def test_quest_read_ratio_worked_example():
    g = json.load(open(os.path.join(GOLD, "quest_read_ratio.json")))
    r = synth.quest_read_ratio(g["page_size"], g["context_tokens"], g["k_pages"])
    assert r == g["ratio"]
    assert g["context_tokens"] // g["page_size"] == g["page_num"]
    # the step-bytes model gives the same ratio on a bf16 layer of that shape
    wl = synth.make_custom(B=1, Hq=1, Hkv=1, lens=(g["context_tokens"],), kv_dtype="bf16",
                           budget_pages=g["k_pages"], n_head_forced=0, n_tail_forced=0)
    sb = synth.step_bytes(wl)
    dense_kv = synth.dense_bytes(wl) - sb["q"] - sb["out"]
    assert (sb["meta"] + sb["kv"]) / dense_kv == g["ratio"]


def test_kv_cache_size_examples():
    g = json.load(open(os.path.join(GOLD, "kv_cache_sizes.json")))
    for c in g["cases"]:
        assert synth.kv_cache_bytes(c["n_layer"], c["context_tokens"], c["n_kv_head"], c["d_head"],
                                    c["elt_bytes"]) == c["bytes"]


def test_headline_step_bytes():
    # one layer of the 16 GB Llama-7B cache: 512 MiB of K+V; 128-page budget
    wl = synth.make_custom(B=1, Hq=32, Hkv=32, lens=(32768,), kv_dtype="bf16", budget_pages=128)
    sb = synth.step_bytes(wl)
    assert synth.dense_bytes(wl) - sb["q"] - sb["out"] == 512 << 20
    assert sb["meta"] == 32 << 20 and sb["kv"] == 32 << 20
    assert sb["q"] + sb["out"] == 24 << 10
