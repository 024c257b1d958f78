"""sa_sparse_decode_attn_noalloc, the attention entry point for callers that cannot
allocate (its partial records live in the library's own per-GPU scratch), called
through the C ABI and compared with sa_sparse_decode_attn (caller workspace) on the
same inputs: bit for bit, and within the attention tolerance of the oracle.  Two
calls in a row, the second with a smaller input (fewer sequences, shorter lists,
another group size), then the int8 cache and a dense pass (run on an MI355X)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import query_aware_sparse_min_amd as sa
import synth
from sa_testlib import GpuCase, check_attention

pytestmark = pytest.mark.gpu


def _noalloc(c, sel, num):
    wl = c.wl
    out = torch.full((wl.B, wl.Hq, wl.d), float("nan"), dtype=torch.float32, device=c.dev)
    vp = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())  # noqa: E731
    rc = sa.load().sa_sparse_decode_attn_noalloc(
        vp(c.d.q), sa._dtype_code(c.d.q), wl.Hq, ctypes.byref(c.kv.struct()),
        ctypes.byref(c.seqs.struct()), vp(sel), vp(num), 0 if sel is None else sel.shape[-1],
        wl.softmax_scale, vp(out), ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == sa.SA_OK, sa.status_string(rc)
    return out


def _compare(wl, dense=False):
    print(f"[gpu] noalloc: B={wl.B} Hq={wl.Hq} Hkv={wl.Hkv} lens={list(wl.seq_lens)} "
          f"kv={wl.kv_dtype} dense={dense}", flush=True)
    c = GpuCase(wl)
    if dense:
        sel = num = None
        o_sel = o_num = None
    else:
        c.build_meta()
        sel, num = c.topk(c.scores())
        o_sel, o_num = sel.cpu().numpy(), num.cpu().numpy()
    ref = c.attention(sel, num)
    out = _noalloc(c, sel, num)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), "differs from the workspace entry point"
    o_out = oracle.attention(wl.q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale,
                             wl.page_table, wl.seq_lens, o_sel, o_num, wl.softmax_scale)
    err = check_attention(wl, out.cpu().numpy(), o_out, what="noalloc attention")
    print(f"[gpu] noalloc ok (err {err:.2e})", flush=True)


def test_noalloc_attention_matches_workspace_entry_point():
    big = synth.make_custom(B=4, Hq=16, Hkv=4, lens=(6000, 3001, 16 * 200, 777), kv_dtype="bf16",
                            q_dtype="bf16", budget_pages=48, page_table="random", seed=81)
    small = synth.make_custom(B=2, Hq=4, Hkv=2, lens=(900, 33), kv_dtype="bf16", q_dtype="bf16",
                              budget_pages=8, page_table="random", seed=82)
    _compare(big)
    _compare(small)  # the scratch keeps the previous call's records: nothing may depend on them
    i8 = synth.make_custom(B=2, Hq=8, Hkv=2, lens=(3000, 1200), kv_dtype="i8", q_dtype="bf16",
                           mode="sals", k_compete=6, page_table="random", seed=83)
    _compare(i8)
    dense = synth.make_custom(B=3, Hq=8, Hkv=8, lens=(5000, 100, 2600), kv_dtype="bf16",
                              q_dtype="bf16", page_table="random", seed=84)
    _compare(dense, dense=True)
