"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it with the CPU oracle on the same seeded inputs.

Tolerances (stated by the method's target and derived in the design notes):
  * metadata, int4 index codes/scales, selections on identical scores: bit-exact;
  * scores: |gpu - oracle| <= 2e-6 * max(|oracle|, A), A = the oracle's absolute
    magnitude of the summed terms (fp32 tree sums of <= 256 terms);
  * selection vs the oracle's selection: equal, except order swaps across the
    k-th boundary between units whose oracle scores differ by at most
    1e-6 * max(|a|, |b|, A_a, A_b);
  * attention: 2e-3 absolute (fp32 output from fp32/bf16 inputs), 8e-3 on int8 KV.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle
import query_aware_sparse_min_amd as sa
import synth

SCORE_RTOL = 2e-6
SWAP_RTOL = 1e-6


def attn_tol(wl) -> float:
    return 8e-3 if wl.kv_dtype == "i8" else 2e-3


class GpuCase:
    """Device copies of a workload plus the binding's argument objects."""

    def __init__(self, wl, device="cuda"):
        self.wl = wl
        self.dev = torch.device(device)
        self.d = synth.to_device(wl, self.dev)
        self.kv = sa.KVCache(self.d.k, self.d.v, self.d.k_scale, self.d.v_scale)
        self.seqs = sa.Seqs(self.d.page_table, self.d.seq_lens)
        mode = {"quest": sa.SA_MODE_QUEST, "sals": sa.SA_MODE_SALS, "probe": sa.SA_MODE_PROBE}[wl.mode]
        self.cfg = sa.SelectCfg(mode, wl.unit_tokens, wl.k_compete, wl.n_head_forced,
                                wl.n_tail_forced, wl.rank, self.d.proj, wl.lse_scale, wl.n_probe)
        self.meta = self.meta_scale = None

    # -- steps -------------------------------------------------------------
    def build_meta(self):
        self.meta, self.meta_scale = sa.alloc_meta(self.kv, self.cfg)
        sa.sa_build_page_meta(self.kv, self.seqs, self.cfg, self.meta, self.meta_scale)
        return self.meta, self.meta_scale

    def q(self, q_np=None):
        return self.d.q if q_np is None else synth.q_to_device(self.wl, q_np, self.dev)

    def scores(self, q_np=None):
        mu = sa.sa_max_units(self.seqs, self.cfg)
        sc = torch.full((self.wl.B, self.wl.Hkv, mu), float("nan"), dtype=torch.float32, device=self.dev)
        sa.sa_score_pages(self.q(q_np), self.kv, self.seqs, self.cfg, self.meta, self.meta_scale, sc)
        return sc

    def topk(self, scores_t):
        ms = sa.sa_max_selected(self.seqs, self.cfg)
        sel = torch.full((self.wl.B, self.wl.Hkv, ms), -7, dtype=torch.int32, device=self.dev)
        num = torch.full((self.wl.B, self.wl.Hkv), -7, dtype=torch.int32, device=self.dev)
        sa.sa_topk_pages(scores_t, self.wl.Hkv, self.seqs, self.cfg, sel, num)
        return sel, num

    def attention(self, sel, num, q_np=None):
        wl = self.wl
        max_sel = 0 if sel is None else sel.shape[-1]
        ws = sa.alloc_workspace(sa.sa_attn_workspace_size(wl.B, wl.Hq, wl.Hkv, wl.max_pages, max_sel),
                                self.dev)
        out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=self.dev)
        sa.sa_sparse_decode_attn(self.q(q_np), self.kv, self.seqs, sel, num, wl.softmax_scale, out, ws)
        return out

    def step(self, q_np=None, want_sel=True):
        wl = self.wl
        ws = sa.alloc_workspace(sa.sa_decode_step_workspace_size(wl.Hq, self.kv, self.seqs, self.cfg),
                                self.dev)
        out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=self.dev)
        sel = num = None
        if want_sel:  # one list per kv-head, or per query head with per-head selection
            ms = sa.sa_max_selected(self.seqs, self.cfg)
            lists = wl.Hq if self.cfg.per_head else wl.Hkv
            sel = torch.full((wl.B, lists, ms), -7, dtype=torch.int32, device=self.dev)
            num = torch.full((wl.B, lists), -7, dtype=torch.int32, device=self.dev)
        sa.sa_decode_step(self.q(q_np), self.kv, self.seqs, self.cfg, self.meta, self.meta_scale,
                          wl.softmax_scale, out, ws, sel, num)
        assert_handoff_words_clear(ws, wl.B * wl.Hkv)
        return out, sel, num


def assert_handoff_words_clear(ws: torch.Tensor, lists: int) -> None:
    """After a completed decode step its workspace's per-list arrival counters (the
    first words; only the fused kernel writes them) are zero again."""
    assert int(torch.count_nonzero(ws[:4 * lists])) == 0, "arrival counters not returned to zero"


def np_u16(t: torch.Tensor) -> np.ndarray:
    """Raw 16-bit words of a bf16 / int16 tensor as uint16."""
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def meta_np(case: GpuCase):
    m = case.meta
    if case.wl.mode == "probe":  # no metadata: the scores read K
        return None, None
    if case.wl.mode == "quest":
        return (m.cpu().numpy() if m.dtype == torch.float32 else np_u16(m)), None
    return m.cpu().numpy(), np_u16(case.meta_scale)


# -- comparisons ------------------------------------------------------------
def check_scores(wl, g_sc: np.ndarray, o_sc: np.ndarray, o_ab: np.ndarray):
    for b in range(wl.B):
        n = wl.n_units(b)
        g, o, a = g_sc[b, :, :n], o_sc[b, :, :n], o_ab[b, :, :n]
        assert np.all(np.isfinite(g)), f"non-finite GPU score (b={b})"
        err = np.abs(g.astype(np.float64) - o)
        bound = SCORE_RTOL * np.maximum(np.abs(o), a)
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), (f"score mismatch b={b} h,u={worst}: gpu={g[worst]!r} "
                                      f"oracle={o[worst]!r} bound={bound[worst]:.3g}")


def check_selection(wl, g_sel, g_num, o_sel, o_num, o_sc, o_ab):
    """GPU selection equals the oracle's up to near-tie swaps at the k-th boundary.
    Returns the set of (b, h) lists that differ (by permitted swaps only)."""
    upu = wl.unit_pages
    swapped = set()
    for b in range(wl.B):
        n = wl.n_units(b)
        for h in range(wl.Hkv):
            gs = list(g_sel[b, h, :g_num[b, h]])
            os_ = list(o_sel[b, h, :o_num[b, h]])
            assert g_num[b, h] == o_num[b, h], f"count differs at b={b} h={h}: {g_num[b, h]} vs {o_num[b, h]}"
            assert np.all(g_sel[b, h, g_num[b, h]:] == -1), "unused selection slots must be -1"
            if gs == os_:
                continue
            assert gs == sorted(gs) and len(set(gs)) == len(gs), "selection not ascending/unique"
            gu = {p // upu for p in gs}
            ou = {p // upu for p in os_}
            only_g, only_o = gu - ou, ou - gu
            mid = set(range(wl.n_head_forced, n - wl.n_tail_forced))
            assert only_g <= mid and only_o <= mid and len(only_g) == len(only_o)
            sc, ab = o_sc[b, h], o_ab[b, h]
            kept = sorted((sc[u] for u in ou & mid), reverse=False)
            s_k = kept[0] if kept else -np.inf  # oracle's k-th best middle score
            for u in only_g | only_o:
                tol = SWAP_RTOL * max(abs(sc[u]), abs(s_k), ab[u])
                assert abs(sc[u] - s_k) <= tol, (f"illegal selection swap b={b} h={h} unit={u}: "
                                                 f"score {sc[u]!r} vs boundary {s_k!r}")
            swapped.add((b, h))
    return swapped


def check_attention(wl, g_out: np.ndarray, o_out: np.ndarray, rows=None, what="attention"):
    g = g_out.reshape(-1, wl.d)
    if rows is not None:
        g = g[rows]
    o = o_out.reshape(-1, wl.d)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g.astype(np.float64) - o)
    assert err.max() <= attn_tol(wl), f"{what}: max |gpu - oracle| = {err.max():.3e}"
    return float(err.max())


def oracle_rows_for_lists(wl, lists):
    """Flattened (b * Hq + head) rows of the query heads of the given (b, h) lists."""
    return np.array(sorted(b * wl.Hq + h * wl.G + g for (b, h) in lists for g in range(wl.G)),
                    dtype=np.int32)
