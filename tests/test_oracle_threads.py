"""The oracle's OpenMP outer loops (one output per iteration) give bit-identical
results at any thread count: metadata, scores, selection and attention of a
GQA workload with a random page table, and the SALS index and block scores."""
import numpy as np

import oracle
import synth


def _step(wl, threads):
    oracle.set_threads(threads)
    try:
        meta, ms = oracle.build_meta(wl)
        out, sel, num, sc, ab = oracle.decode_step(wl, meta, ms)
        return meta, ms, out, sel, num, sc, ab
    finally:
        oracle.set_threads(1)


def test_thread_count_does_not_change_results():
    for kw in (dict(B=3, Hq=8, Hkv=2, lens=(3000, 17, 1600), kv_dtype="bf16", q_dtype="bf16",
                    budget_pages=20, page_table="random"),
               dict(B=2, Hq=8, Hkv=2, lens=(2000, 900), kv_dtype="i8", q_dtype="bf16", mode="sals",
                    k_compete=6, page_table="random")):
        wl = synth.make_custom(**kw, seed=91)
        one, four = _step(wl, 1), _step(wl, 4)
        for a, b in zip(one, four):
            if a is None:
                assert b is None
                continue
            assert a.dtype == b.dtype and np.array_equal(a.view(np.uint8), b.view(np.uint8))
