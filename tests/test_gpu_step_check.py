"""The fused decode step's hand-offs (run on an MI355X).

* A Quest step with one query head per kv-head runs as the fused persistent
  kernel: that kernel returns its per-list arrival counters and score-key
  words to zero, while the separate kernels leave fp32 scores in the score
  region, so an all-zero counter and key region after the call shows that the
  fused kernel ran (its build uses no scratch memory).  Workspace layout: the
  counters (one word per list, padded to 256 bytes), then one key row of
  max_pages words per list.
* No workgroup of the fused kernel waits for another one: with its grid capped
  at a few workgroups (SA_STEP_MAX_WORKGROUPS), most chunks of a list are not
  resident while its first chunk runs, so that chunk scores the other chunks'
  pages itself after its bounded wait.  The output, the page lists and the
  cleared workspace must equal those of the full grid bit for bit.
* The same holds for the persistent selection + attention + merge kernel that
  follows a separate scorer (SALS on an int8 cache, Quest with GQA groups):
  capped at one or a few workgroups, output and page lists are bit-identical
  and the arrival counters return to zero.
"""
import os

import pytest
import torch

import query_aware_sparse_min_amd as sa
import synth
from sa_testlib import GpuCase

pytestmark = pytest.mark.gpu


def _case():
    wl = synth.make_custom(B=2, Hq=8, Hkv=8, lens=(16 * 600 - 5, 16 * 430), kv_dtype="bf16",
                           q_dtype="bf16", budget_pages=20, page_table="random", seed=71)
    c = GpuCase(wl)
    c.build_meta()
    return wl, c


def _handoff_region(wl, ws):
    lists = wl.B * wl.Hkv
    return ws[:-(-4 * lists // 256) * 256 + 4 * lists * wl.max_pages]


def _run(c, wl, ws, want_sel=True):
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=c.dev)
    ms = sa.sa_max_selected(c.seqs, c.cfg)
    sel = torch.full((wl.B, wl.Hkv, ms), -7, dtype=torch.int32, device=c.dev) if want_sel else None
    num = torch.full((wl.B, wl.Hkv), -7, dtype=torch.int32, device=c.dev) if want_sel else None
    sa.sa_decode_step(c.d.q, c.kv, c.seqs, c.cfg, c.meta, c.meta_scale, wl.softmax_scale, out, ws, sel, num)
    torch.cuda.synchronize()
    return out, sel, num


def test_fused_step_runs_and_clears_its_hand_off_words():
    wl, c = _case()
    print("[gpu] fused step launch check", flush=True)
    ws = sa.alloc_workspace(sa.sa_decode_step_workspace_size(wl.Hq, c.kv, c.seqs, c.cfg), c.dev)
    ref = None
    for _ in range(3):
        out, sel, num = _run(c, wl, ws)
        assert int(torch.count_nonzero(_handoff_region(wl, ws))) == 0, \
            "the separate kernels ran, or hand-off words were left"
        if ref is None:
            ref = (out, sel, num)
        assert torch.equal(out.view(torch.int32), ref[0].view(torch.int32))
        assert torch.equal(sel, ref[1]) and torch.equal(num, ref[2])


@pytest.mark.parametrize("grid", [1, 3, 7])
def test_fused_step_with_few_resident_workgroups(grid):
    wl, c = _case()
    print(f"[gpu] fused step on {grid} workgroups", flush=True)
    ws = sa.alloc_workspace(sa.sa_decode_step_workspace_size(wl.Hq, c.kv, c.seqs, c.cfg), c.dev)
    ref_out, ref_sel, ref_num = _run(c, wl, ws)
    os.environ["SA_STEP_MAX_WORKGROUPS"] = str(grid)
    try:
        for _ in range(2):
            out, sel, num = _run(c, wl, ws)
            assert int(torch.count_nonzero(_handoff_region(wl, ws))) == 0, "hand-off words were left behind"
            assert torch.equal(sel, ref_sel) and torch.equal(num, ref_num)
            assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32))
    finally:
        del os.environ["SA_STEP_MAX_WORKGROUPS"]


@pytest.mark.parametrize("grid", [1, 5])
@pytest.mark.parametrize("kind", ["sals_i8", "gqa4_bf16", "gqa16_bf16", "probe_gqa2"])
def test_post_score_kernel_with_few_resident_workgroups(kind, grid):
    kw = {"sals_i8": dict(B=2, Hq=8, Hkv=2, lens=(5000, 1300), kv_dtype="i8", mode="sals", k_compete=9),
          "gqa4_bf16": dict(B=3, Hq=16, Hkv=4, lens=(4000, 777, 2500), kv_dtype="bf16", budget_pages=40),
          "gqa16_bf16": dict(B=1, Hq=32, Hkv=2, lens=(3000,), kv_dtype="bf16", budget_pages=24),
          "probe_gqa2": dict(B=2, Hq=8, Hkv=4, lens=(2000, 900), kv_dtype="bf16", mode="probe",
                             k_compete=10)}[kind]
    wl = synth.make_custom(q_dtype="bf16", page_table="random", seed=72, **kw)
    c = GpuCase(wl)
    c.build_meta()
    print(f"[gpu] post-score kernel {kind} on {grid} workgroups", flush=True)
    ws = sa.alloc_workspace(sa.sa_decode_step_workspace_size(wl.Hq, c.kv, c.seqs, c.cfg), c.dev)
    ref_out, ref_sel, ref_num = _run(c, wl, ws)
    os.environ["SA_STEP_MAX_WORKGROUPS"] = str(grid)
    try:
        out, sel, num = _run(c, wl, ws)
    finally:
        del os.environ["SA_STEP_MAX_WORKGROUPS"]
    assert int(torch.count_nonzero(ws[:4 * wl.B * wl.Hkv])) == 0, "arrival counters left behind"
    assert torch.equal(sel, ref_sel) and torch.equal(num, ref_num)
    assert torch.equal(out.view(torch.int32), ref_out.view(torch.int32))

