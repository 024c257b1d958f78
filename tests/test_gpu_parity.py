"""GPU-vs-oracle parity of every step through the C ABI, on small seeded
workloads that span several tiles and ragged tails (run on an MI355X)."""
import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_min_amd as sa
import synth
from sa_testlib import (GpuCase, assert_handoff_words_clear, attn_tol, check_attention,
                        check_scores, check_selection, meta_np, oracle_rows_for_lists)

pytestmark = pytest.mark.gpu

CASES = {
    "mha_f32": dict(B=1, Hq=8, Hkv=8, lens=(2048,), kv_dtype="f32", q_dtype="f32", budget_pages=16),
    "mha_bf16_ragged": dict(B=3, Hq=4, Hkv=4, lens=(1000, 17, 3333), kv_dtype="bf16",
                            q_dtype="bf16", budget_pages=24, page_table="random"),
    "gqa2_bf16kv_f32q": dict(B=2, Hq=8, Hkv=4, lens=(1500, 700), kv_dtype="bf16", q_dtype="f32",
                             budget_pages=20, page_table="random"),
    "gqa4_bf16": dict(B=4, Hq=16, Hkv=4, lens=(3000, 300, 2047, 1025), kv_dtype="bf16",
                      q_dtype="bf16", budget_pages=32, page_table="random"),
    "gqa8_bf16": dict(B=2, Hq=16, Hkv=2, lens=(4096, 2500), kv_dtype="bf16", q_dtype="bf16",
                      budget_pages=40),
    "gqa16_bf16": dict(B=1, Hq=32, Hkv=2, lens=(2222,), kv_dtype="bf16", q_dtype="bf16",
                       budget_pages=20),
    "gqa4_f32": dict(B=2, Hq=8, Hkv=2, lens=(900, 1601), kv_dtype="f32", q_dtype="f32",
                     budget_pages=12, page_table="random"),
    "sals_i8": dict(B=2, Hq=8, Hkv=2, lens=(5000, 700), kv_dtype="i8", q_dtype="bf16", mode="sals",
                    k_compete=8, page_table="random"),
    "sals_bf16": dict(B=2, Hq=32, Hkv=8, lens=(4100, 1000), kv_dtype="bf16", q_dtype="bf16",
                      mode="sals", k_compete=6),
    "sals_f32_h1": dict(B=1, Hq=4, Hkv=1, lens=(3000,), kv_dtype="f32", q_dtype="f32",
                        mode="sals", k_compete=5),
    "sals_i8_h16": dict(B=1, Hq=16, Hkv=16, lens=(2100,), kv_dtype="i8", q_dtype="bf16",
                        mode="sals", k_compete=4),
    # many lists x pages, B = 2, ragged: several chunks per list and empty chunks
    "mha_bf16_b2_long": dict(B=2, Hq=16, Hkv=16, lens=(16384, 9000), kv_dtype="bf16",
                               q_dtype="bf16", budget_pages=40, page_table="random"),
    # probe sampling: 32-token blocks with 8 probes (step 4), 64-token blocks, 16-token
    # blocks with 5 probes (step 3: six probes), and 12 probes of 32 (step 2: two rounds)
    "probe_bf16": dict(B=2, Hq=8, Hkv=8, lens=(2000, 777), kv_dtype="bf16", q_dtype="bf16",
                       mode="probe", k_compete=12, page_table="random"),
    "probe_gqa4_i8": dict(B=2, Hq=16, Hkv=4, lens=(3000, 1234), kv_dtype="i8", q_dtype="bf16",
                          mode="probe", unit_tokens=64, k_compete=6, page_table="random"),
    "probe_f32_u16": dict(B=1, Hq=2, Hkv=1, lens=(1500,), kv_dtype="f32", q_dtype="f32",
                          mode="probe", unit_tokens=16, n_probe=5, k_compete=20),
    "probe_gqa8_p12": dict(B=1, Hq=16, Hkv=2, lens=(2500,), kv_dtype="bf16", q_dtype="bf16",
                           mode="probe", n_probe=12, k_compete=10),
    # a list of 18750 pages: the top-K that re-reads its keys from the scores
    "gqa2_bf16_18k_pages": dict(B=1, Hq=2, Hkv=1, lens=(300000,), kv_dtype="bf16",
                                q_dtype="bf16", budget_pages=64),
    # the fused step with lists of 2049..4096 pages (eight register keys per thread):
    # one query head per kv-head, Quest, random page tables, bf16 and fp32
    "mha_bf16_64k_kpt_hi": dict(B=2, Hq=2, Hkv=2, lens=(65536, 40000), kv_dtype="bf16",
                                q_dtype="bf16", budget_pages=200, page_table="random"),
    "mha_f32_64k_kpt_hi": dict(B=2, Hq=2, Hkv=2, lens=(65536, 40000), kv_dtype="f32",
                               q_dtype="f32", budget_pages=130, page_table="random"),
}


def _full_check(wl, label):
    print(f"[gpu] case {label}: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} lens={list(wl.seq_lens)} "
          f"kv={wl.kv_dtype} mode={wl.mode}", flush=True)
    c = GpuCase(wl)
    c.build_meta()
    o_meta, o_ms = oracle.build_meta(wl)
    g_meta, g_ms = meta_np(c)
    # metadata / index key: bit-exact on every referenced page
    for b in range(wl.B):
        pages = wl.page_table[b, :wl.n_pages(b)]
        if wl.mode == "quest":  # [Hkv, P, 2, d]
            assert np.array_equal(g_meta[:, pages].view(np.uint8), o_meta[:, pages].view(np.uint8)), \
                f"metadata differs (b={b})"
        elif wl.mode == "sals":  # codes [P, S, Hkv, r/2], scales [P, S, Hkv]
            assert np.array_equal(g_meta[pages], o_meta[pages]), f"index codes differ (b={b})"
            assert np.array_equal(g_ms[pages], o_ms[pages]), f"index scales differ (b={b})"
    # scores
    g_sc_t = c.scores()
    g_sc = g_sc_t.cpu().numpy()
    o_sc, o_ab = oracle.score(wl, o_meta, o_ms)
    check_scores(wl, g_sc, o_sc, o_ab)
    # selection on identical (GPU) scores: bit-exact
    g_sel_t, g_num_t = c.topk(g_sc_t)
    g_sel, g_num = g_sel_t.cpu().numpy(), g_num_t.cpu().numpy()
    r_sel, r_num = oracle.select(np.where(np.isnan(g_sc), -np.inf, g_sc).astype(np.float64),
                                 wl.seq_lens, wl.unit_tokens, wl.k_compete, wl.n_head_forced,
                                 wl.n_tail_forced, wl.max_sel)
    assert np.array_equal(g_num, r_num) and np.array_equal(g_sel, r_sel), "top-K differs on identical scores"
    # selection vs the oracle's own scores
    o_sel, o_num = oracle.select(o_sc, wl.seq_lens, wl.unit_tokens, wl.k_compete, wl.n_head_forced,
                                 wl.n_tail_forced, wl.max_sel)
    swapped = check_selection(wl, g_sel, g_num, o_sel, o_num, o_sc, o_ab)
    # attention on the oracle's selection
    o_out = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale,
                             wl.page_table, wl.seq_lens, o_sel, o_num, wl.softmax_scale)
    g_out = c.attention(torch.from_numpy(o_sel).to(c.dev), torch.from_numpy(o_num).to(c.dev))
    e_attn = check_attention(wl, g_out.cpu().numpy(), o_out, what="sparse attention")
    # fused step: rows of lists whose selection matches the oracle's are compared with the
    # oracle; lists with a permitted near-tie swap are compared with the GPU attention kernel
    # run on the step's own selection
    s_out, s_sel, s_num = c.step()
    s_out, s_sel, s_num = s_out.cpu().numpy(), s_sel.cpu().numpy(), s_num.cpu().numpy()
    assert np.array_equal(s_sel, g_sel) and np.array_equal(s_num, g_num), "step selection differs"
    keep = [(b, h) for b in range(wl.B) for h in range(wl.Hkv) if (b, h) not in swapped]
    rows = oracle_rows_for_lists(wl, keep)
    if len(rows):
        check_attention(wl, s_out, o_out.reshape(-1, wl.d)[rows], rows=rows, what="decode step")
    if swapped:
        rows2 = oracle_rows_for_lists(wl, swapped)
        ref = c.attention(torch.from_numpy(s_sel).to(c.dev), torch.from_numpy(s_num).to(c.dev))
        assert np.array_equal(s_out.reshape(-1, wl.d)[rows2], ref.cpu().numpy().reshape(-1, wl.d)[rows2])
    print(f"[gpu] case {label}: ok (attn err {e_attn:.2e}, swapped lists {len(swapped)})", flush=True)
    return c


@pytest.mark.parametrize("label", sorted(CASES))
def test_step_parity(label):
    wl = synth.make_custom(**CASES[label], seed=40 + sorted(CASES).index(label), name=label)
    _full_check(wl, label)


@pytest.mark.parametrize("lens,budget", [((1,), 16), ((16,), 16), ((17,), 2), ((15, 33, 48), 2),
                                         ((300,), 2), ((16 * 40 + 1,), 3)])
def test_short_and_edge_lengths(lens, budget):
    wl = synth.make_custom(B=len(lens), Hq=4, Hkv=2, lens=lens, kv_dtype="bf16", q_dtype="bf16",
                           budget_pages=budget, page_table="random", seed=3)
    _full_check(wl, f"edge{lens}/{budget}")


def test_only_forced_units():
    wl = synth.make_custom(B=2, Hq=8, Hkv=4, lens=(1111, 640), kv_dtype="bf16", q_dtype="bf16",
                           k_compete=0, page_table="random", seed=5)
    _full_check(wl, "k0")


def test_sals_with_sink_and_partial_last_block():
    wl = synth.make_custom(B=2, Hq=8, Hkv=4, lens=(64 * 30 + 20, 64 * 3 + 1), kv_dtype="i8",
                           q_dtype="bf16", mode="sals", k_compete=3, n_head_forced=1,
                           n_tail_forced=1, seed=6)
    _full_check(wl, "sals_sink")


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16", "i8"])
def test_dense_attention_matches_oracle(kv_dtype):
    wl = synth.make_custom(B=3, Hq=8, Hkv=2, lens=(2000, 1, 777), kv_dtype=kv_dtype,
                           q_dtype="bf16", page_table="random", seed=8,
                           mode="sals" if kv_dtype == "i8" else "quest")
    print(f"[gpu] dense attention {kv_dtype}", flush=True)
    c = GpuCase(wl)
    g = c.attention(None, None).cpu().numpy()
    o = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale,
                         wl.page_table, wl.seq_lens, None, None, wl.softmax_scale)
    check_attention(wl, g, o, what="dense attention")


@pytest.mark.parametrize("shape", ["many_uneven", "one_long", "past_plan_limit"])
def test_dense_ragged_batches(shape):
    """Dense passes over batches of very uneven lengths (empty sequences included):
    the device split plan cuts each list by its own length.  past_plan_limit has
    more sequences than the device plan takes, so the host plan runs instead."""
    rng = np.random.default_rng({"many_uneven": 31, "one_long": 32, "past_plan_limit": 33}[shape])
    if shape == "many_uneven":
        lens = rng.choice([0, 1, 15, 16, 17, 100, 555, 2000, 6000], size=300)
        kw = dict(Hq=8, Hkv=2, kv_dtype="bf16")
    elif shape == "one_long":
        lens = np.array([65536, 1, 0, 33, 16])
        kw = dict(Hq=16, Hkv=8, kv_dtype="i8", mode="sals")
    else:
        lens = rng.integers(0, 48, size=1100)
        kw = dict(Hq=4, Hkv=4, kv_dtype="f32")
    wl = synth.make_custom(B=len(lens), lens=tuple(int(x) for x in lens), q_dtype="bf16",
                           page_table="random", seed=34, **kw)
    print(f"[gpu] dense ragged {shape}: B={wl.B} pages={sum(wl.n_pages(b) for b in range(wl.B))}",
          flush=True)
    c = GpuCase(wl)
    g = c.attention(None, None).cpu().numpy()
    o = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale,
                         wl.page_table, wl.seq_lens, None, None, wl.softmax_scale)
    check_attention(wl, g, o, what=f"dense ragged {shape}")
    assert np.all(g[np.asarray(lens) == 0] == 0.0), "an empty sequence attends to nothing"


def test_all_pages_budget_equals_dense():
    """Budget >= every unit: the step skips scoring and equals dense attention."""
    wl = synth.make_custom(B=2, Hq=16, Hkv=4, lens=(3000, 2000), kv_dtype="bf16", q_dtype="bf16",
                           budget_pages=10 ** 4, page_table="random", seed=9)
    c = GpuCase(wl)
    c.build_meta()
    out, sel, num = c.step()
    dense = c.attention(None, None)
    assert torch.equal(out, dense)
    for b in range(2):
        assert np.all(num.cpu().numpy()[b] == wl.n_pages(b))
    o = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, None, None, wl.page_table,
                         wl.seq_lens, None, None, wl.softmax_scale)
    check_attention(wl, out.cpu().numpy(), o, what="all-pages step")


def test_repeated_runs_are_bit_identical():
    wl = synth.make_custom(B=2, Hq=16, Hkv=4, lens=(5000, 3000), kv_dtype="bf16", q_dtype="bf16",
                           budget_pages=64, page_table="random", seed=10)
    c = GpuCase(wl)
    c.build_meta()
    o1, s1, n1 = c.step()
    o2, s2, n2 = c.step()
    assert torch.equal(s1, s2) and torch.equal(n1, n2)
    assert torch.equal(o1.view(torch.int32), o2.view(torch.int32))


@pytest.mark.parametrize("kv_dtype", ["f32", "bf16"])
def test_strong_needle_is_selected(kv_dtype):
    """A needle whose true dot beats every other page's bound must be selected."""
    wl = synth.make_custom(B=1, Hq=4, Hkv=4, lens=(16 * 200 - 5,), kv_dtype=kv_dtype,
                           q_dtype=kv_dtype, budget_pages=4, seed=12)
    o_meta, _ = oracle.build_meta(wl)
    sc, _ = oracle.score(wl, o_meta, None)
    n = wl.n_pages(0)
    Q = (synth.bf16_to_f32(wl.q) if kv_dtype == "bf16" else wl.q).astype(np.float64)
    pages = synth.uniform_int(1, 77, 4, 1, n - 2)
    for h in range(4):
        p = int(pages[h])
        others = np.delete(sc[0, h, 1:n - 1], p - 1)
        qn = np.linalg.norm(Q[0, h])
        key = (1.25 * max(others.max(), 1e-3) / qn * Q[0, h] / qn).astype(np.float32)
        wl.k[p, 3, h] = key if kv_dtype == "f32" else synth.f32_to_bf16(key)
    c = GpuCase(wl)
    c.build_meta()
    _, sel, num = c.step()
    sel, num = sel.cpu().numpy(), num.cpu().numpy()
    for h in range(4):
        assert int(pages[h]) in sel[0, h, :num[0, h]]


# ---------------------------------------------------------------- top-K alone
def _topk_case(lens, mu, k, fh, ft, ut, scores):
    import query_aware_sparse_min_amd as sa
    dev = torch.device("cuda")
    B = len(lens)
    max_pages = -(-mu * ut // 16)
    lens = np.array([min(L, max_pages * 16) for L in lens], dtype=np.int32)
    seqs = sa.Seqs(torch.zeros((B, max_pages), dtype=torch.int32, device=dev),
                   torch.from_numpy(lens).to(dev))
    cfg = sa.SelectCfg(sa.SA_MODE_QUEST if ut == 16 else sa.SA_MODE_SALS, ut, k, fh, ft)
    ms = sa.sa_max_selected(seqs, cfg)
    sel = torch.full((B, 1, ms), -7, dtype=torch.int32, device=dev)
    num = torch.full((B, 1), -7, dtype=torch.int32, device=dev)
    sa.sa_topk_pages(torch.from_numpy(scores.astype(np.float32)).to(dev), 1, seqs, cfg, sel, num)
    o_sel, o_num = oracle.select(scores.astype(np.float32).astype(np.float64), lens, ut, k, fh, ft, ms)
    assert np.array_equal(num.cpu().numpy(), o_num)
    assert np.array_equal(sel.cpu().numpy(), o_sel)


@pytest.mark.parametrize("n,k", [(40, 5), (3000, 126), (16384, 254), (20000, 300), (5000, 4990)])
def test_topk_bit_exact_with_ties(n, k):
    rng = np.random.default_rng(n)
    vals = np.array([-3.0, -0.0, 0.0, 1.5, 1.5000001, 7.0, -np.inf], dtype=np.float32)
    sc = rng.choice(vals, size=(2, 1, n)).astype(np.float32)
    sc[1, 0] = rng.standard_normal(n).astype(np.float32)
    sc[1, 0, ::7] = sc[1, 0, 3]  # exact ties in a continuous spread
    print(f"[gpu] topk n={n} k={k}", flush=True)
    _topk_case((n * 16, n * 16 - 9), n, k, 1, 1, 16, sc)


def test_topk_all_equal_and_sals_units():
    n = 1000
    sc = np.full((1, 1, n), 2.5, dtype=np.float32)
    _topk_case((n * 16,), n, 100, 1, 1, 16, sc)
    rng = np.random.default_rng(3)
    sc = rng.standard_normal((3, 1, 300)).astype(np.float32)
    _topk_case((300 * 64, 299 * 64 + 5, 40 * 64), 300, 32, 0, 2, 64, sc)
    _topk_case((300 * 64, 299 * 64 + 5, 40 * 64), 300, 10, 0, 0, 64, sc)


@pytest.mark.parametrize("gqa", [False, True])
def test_step_graph_replays_match_eager(gqa):
    """The step captured in a HIP graph: every replay (with eager work between replays)
    reproduces the eager result bit for bit; no memset nodes are involved.  MHA runs the
    fused step; GQA-4 runs the scorer, top-K, attention and merge kernels."""
    if gqa:
        wl = synth.make_custom(B=2, Hq=16, Hkv=4, lens=(16 * 300 - 3, 2000), kv_dtype="bf16",
                               q_dtype="bf16", budget_pages=24, page_table="random", seed=14)
    else:
        wl = synth.make_custom(B=1, Hq=8, Hkv=8, lens=(16 * 300 - 3,), kv_dtype="bf16",
                               q_dtype="bf16", budget_pages=24, seed=13)
    c = GpuCase(wl)
    c.build_meta()
    ref_out, ref_sel, ref_num = c.step()
    ws = sa.alloc_workspace(sa.sa_decode_step_workspace_size(wl.Hq, c.kv, c.seqs, c.cfg), c.dev)
    out = torch.zeros((wl.B, wl.Hq, wl.d), dtype=torch.float32, device=c.dev)
    sel = torch.zeros_like(ref_sel)
    num = torch.zeros_like(ref_num)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sa.sa_decode_step(c.d.q, c.kv, c.seqs, c.cfg, c.meta, None, wl.softmax_scale, out, ws,
                              sel, num)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(4):
        out.fill_(float("nan"))
        sel.fill_(-5)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel, ref_sel) and torch.equal(num, ref_num), f"replay {rep}: selection"
        assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32)), f"replay {rep}: output"
        assert_handoff_words_clear(ws, wl.B * wl.Hkv)
        c.step()  # eager work between replays


def test_dense_ragged_graph_replays_match_eager():
    """The device-planned dense pass captured in a HIP graph: every replay, with eager
    work and new sequence lengths between replays, equals the eager call on the same
    lengths bit for bit (the plan is read from the lengths at run time)."""
    wl = synth.make_custom(B=5, Hq=8, Hkv=2, lens=(4000, 0, 17, 2500, 900), kv_dtype="bf16",
                           q_dtype="bf16", page_table="random", seed=35)
    print("[gpu] dense ragged graph replay", flush=True)
    c = GpuCase(wl)
    ws = sa.alloc_workspace(sa.sa_attn_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.max_pages, 0), c.dev)
    out = torch.zeros((wl.B, wl.Hq, wl.d), dtype=torch.float32, device=c.dev)
    lens_t = c.d.seq_lens
    lens0 = lens_t.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            sa.sa_sparse_decode_attn(c.d.q, c.kv, c.seqs, None, None, wl.softmax_scale, out, ws)
    torch.cuda.current_stream().wait_stream(s)
    variants = [lens0, torch.tensor([3, 4000, 0, 16, 2500], dtype=torch.int32, device=c.dev), lens0]
    for rep, lv in enumerate(variants):
        lens_t.copy_(lv)
        ref = c.attention(None, None)  # eager, same lengths
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {rep}"
    lens_t.copy_(lens0)


def test_attention_workspace_is_reusable():
    """Three split-K attention calls on one workspace, each with a new query, equal
    calls on fresh workspaces bit for bit (no state is carried between calls)."""
    wl = synth.make_custom(B=2, Hq=16, Hkv=4, lens=(3000, 1200), kv_dtype="bf16", q_dtype="bf16",
                           budget_pages=48, page_table="random", seed=12)
    print("[gpu] attention workspace reuse", flush=True)
    c = GpuCase(wl)
    c.build_meta()
    sel, num = c.topk(c.scores())
    ws = sa.alloc_workspace(sa.sa_attn_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.max_pages,
                                                      sel.shape[-1]), c.dev)
    for i in range(3):
        q = synth.fresh_q(wl, i)
        out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=c.dev)
        sa.sa_sparse_decode_attn(c.q(q), c.kv, c.seqs, sel, num, wl.softmax_scale, out, ws)
        ref = c.attention(sel, num, q)
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"call {i} differs"


def _random_case(seed):
    """A seeded random small workload: scoring mode, dtypes, group size, batch, ragged
    lengths (down to a single token), budget and page-table layout."""
    r = np.random.default_rng(1000 + seed)
    mode = ["quest", "sals", "probe"][seed % 3]
    hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    B = int(r.integers(1, 4))
    lens = tuple(int(x) for x in r.integers(1, 5001, B))
    kv = str(r.choice(["f32", "bf16"] if mode == "quest" else ["f32", "bf16", "i8"]))
    qd = str(r.choice(["f32", "bf16"]))
    kw = dict(B=B, Hq=hkv * G, Hkv=hkv, lens=lens, kv_dtype=kv, q_dtype=qd, mode=mode,
              page_table=str(r.choice(["random", "contiguous"])))
    if mode == "quest":
        kw["budget_pages"] = int(r.integers(2, 40))
    elif mode == "sals":
        kw["k_compete"] = int(r.integers(0, 12))
    else:
        kw["unit_tokens"] = int(r.choice([16, 32, 64]))
        kw["n_probe"] = int(r.integers(1, 13))
        kw["k_compete"] = int(r.integers(0, 20))
    return kw


@pytest.mark.parametrize("seed", range(12))
def test_random_workloads(seed):
    kw = _random_case(seed)
    wl = synth.make_custom(**kw, seed=500 + seed, name=f"random{seed}")
    _full_check(wl, f"random{seed}: {kw}")


def test_sals_index_query_rounding_adversarial():
    """The SALS scorer's fixed-point index query against its worst case: every int4
    code saturated at +-7 (written directly into the index buffers), an identity
    projection so that the projected query equals q exactly, one component of q at
    1.0 and the other fifteen just past a half step of a fixed-point grid, with
    signs chosen so that every token's fifteen rounding errors add up with the same
    sign.  The scores must stay within the score tolerance of the oracle's
    double-precision scores.  Emulated on the host, an index query of 22 fractional
    bits misses the tolerance on the heads placed on its grid (2.3e-6 of the score
    scale against 2e-6); 26 bits stay at 1.5e-7 on the heads placed on theirs."""
    Hkv, L = 8, 512
    wl = synth.make_custom(B=1, Hq=Hkv, Hkv=Hkv, lens=(L,), kv_dtype="bf16", q_dtype="f32",
                           mode="sals", k_compete=2, seed=77, name="sals-adversarial")
    rng = np.random.default_rng(77)
    proj = np.zeros((wl.d, 16), dtype=np.float32)
    proj[np.arange(16), np.arange(16)] = 1.0
    sign = rng.choice([-1.0, 1.0], size=(Hkv, 16))
    k = rng.integers(1000, 8000, size=(Hkv, 16)).astype(np.float64)
    q = np.zeros((1, Hkv, wl.d), dtype=np.float32)
    # half the heads just past half steps of a 22-bit grid (2^-21 here), half of a 26-bit
    # one (2^-25)
    step = np.where(np.arange(Hkv) < Hkv // 2, 2.0 ** -21, 2.0 ** -25)[:, None]
    q[0, :, :16] = (sign * (k + 0.5 + 2.0 ** -10) * step).astype(np.float32)
    q[0, :, 0] = sign[:, 0]  # the largest component, 1.0: the grid exponent is 1
    nib = np.where(sign > 0, 7, 9).astype(np.uint8)  # +7 / -7 as two's-complement nibbles
    row = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)  # [Hkv, 8]
    P = wl.num_pages
    codes = np.broadcast_to(row, (P, 16, Hkv, 8)).copy()
    scales = synth.f32_to_f16(rng.uniform(4.0, 12.0, size=(P, 16, Hkv)).astype(np.float32))
    wl.q, wl.proj = q, proj
    print("[gpu] sals adversarial rounding case", flush=True)
    c = GpuCase(wl)
    c.meta = torch.from_numpy(codes).to(c.dev)
    c.meta_scale = torch.from_numpy(scales.view(np.int16)).to(c.dev)
    g_sc = c.scores().cpu().numpy()
    o_sc, o_ab = oracle.sals_scores(q, "f32", codes, scales, proj, wl.page_table, wl.seq_lens,
                                    Hkv, wl.unit_tokens, wl.lse_scale)
    check_scores(wl, g_sc, o_sc, o_ab)
    n = wl.n_units(0)
    rel = np.abs(g_sc[0, :, :n] - o_sc[0, :, :n]) / np.maximum(np.abs(o_sc[0, :, :n]), o_ab[0, :, :n])
    print(f"[gpu] sals adversarial: largest error {rel.max():.2e} of the score scale", flush=True)
