"""Python binding of the gfx950 query-aware sparse decode-attention library.

Argument marshalling only: every call below forwards device pointers, sizes
and the current HIP stream to the C ABI declared in include/sa.h (libsa.so,
hand-written HIP kernels).  PyTorch supplies device memory and streams; no
compute happens here, and there is no fallback path: if libsa.so is missing
or fails to load, every entry point raises.

Layouts (see include/sa.h):
  q [B, Hq, 128] fp32 | bf16;  K, V [P, 16, Hkv, 128] fp32 | bf16 | int8
  (+ fp16 scales [P, 16, Hkv]);  page_table [B, max_pages] int32;
  seq_lens [B] int32;  out [B, Hq, 128] fp32.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA_LIB_PATH: load another build of the library (e.g. the host-sanitizer build)
LIB_PATH = os.environ.get("SA_LIB_PATH") or os.path.join(_HERE, "libsa.so")

SA_OK, SA_ERR_INVALID_ARG, SA_ERR_UNSUPPORTED, SA_ERR_WORKSPACE_TOO_SMALL, SA_ERR_HIP = 0, -1, -2, -3, -4
SA_F32, SA_BF16, SA_I8 = 0, 1, 2
SA_MODE_QUEST, SA_MODE_SALS, SA_MODE_PROBE = 0, 1, 2

_lib = None


class SAError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)} ({status})")
        self.status = status


class sa_kv_cache(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("k_scale", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("dtype", ctypes.c_int32),
                ("num_pages", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32)]


class sa_seqs(ctypes.Structure):
    _fields_ = [("page_table", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p),
                ("batch", ctypes.c_int32), ("max_pages", ctypes.c_int32)]


class sa_select_cfg(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("unit_tokens", ctypes.c_int32),
                ("k_compete", ctypes.c_int32), ("n_head_forced", ctypes.c_int32),
                ("n_tail_forced", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("proj", ctypes.c_void_p), ("lse_scale", ctypes.c_float), ("n_probe", ctypes.c_int32),
                ("per_head", ctypes.c_int32)]


EXPORTS = ["sa_version", "sa_status_string", "sa_meta_bytes", "sa_meta_scale_bytes",
           "sa_build_page_meta", "sa_append_kv", "sa_max_units", "sa_score_pages", "sa_max_selected",
           "sa_topk_pages", "sa_attn_workspace_size", "sa_sparse_decode_attn",
           "sa_attn_heads_workspace_size", "sa_sparse_decode_attn_heads",
           "sa_decode_step_workspace_size", "sa_decode_step", "sa_stream_read",
           "sa_sparse_decode_attn_noalloc"]


def load(path: str = LIB_PATH):
    """Load libsa.so (built by query_aware_sparse_min_amd.build); raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    P, I32, SZ, F, VP = ctypes.POINTER, ctypes.c_int32, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p
    KV, SQ, CF = P(sa_kv_cache), P(sa_seqs), P(sa_select_cfg)
    sig = {
        "sa_version": (ctypes.c_int, []),
        "sa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "sa_meta_bytes": (SZ, [KV, CF]),
        "sa_meta_scale_bytes": (SZ, [KV, CF]),
        "sa_build_page_meta": (ctypes.c_int, [KV, SQ, CF, VP, VP, VP]),
        "sa_append_kv": (ctypes.c_int, [VP, VP, VP, VP, KV, SQ, CF, VP, VP, VP]),
        "sa_max_units": (I32, [SQ, CF]),
        "sa_score_pages": (ctypes.c_int, [VP, I32, I32, KV, SQ, CF, VP, VP, VP, VP]),
        "sa_max_selected": (I32, [SQ, CF]),
        "sa_topk_pages": (ctypes.c_int, [VP, I32, SQ, CF, VP, VP, VP]),
        "sa_attn_workspace_size": (SZ, [I32, I32, I32, I32, I32]),
        "sa_sparse_decode_attn": (ctypes.c_int, [VP, I32, I32, KV, SQ, VP, VP, I32, F, VP, VP, SZ, VP]),
        "sa_attn_heads_workspace_size": (SZ, [I32, I32, I32, I32, I32]),
        "sa_sparse_decode_attn_heads": (ctypes.c_int, [VP, I32, I32, KV, SQ, VP, VP, I32, F, VP, VP, SZ, VP]),
        "sa_decode_step_workspace_size": (SZ, [I32, KV, SQ, CF]),
        "sa_decode_step": (ctypes.c_int, [VP, I32, I32, KV, SQ, CF, VP, VP, F, VP, VP, VP, VP, SZ, VP]),
        "sa_stream_read": (ctypes.c_int, [VP, SZ, VP, SZ, VP]),
        "sa_sparse_decode_attn_noalloc": (ctypes.c_int, [VP, I32, I32, KV, SQ, VP, VP, I32, F, VP, VP]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().sa_status_string(status).decode()


def _check(rc: int, where: str) -> None:
    if rc != SA_OK:
        raise SAError(rc, where)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SA_F32
    if t.dtype == torch.bfloat16:
        return SA_BF16
    if t.dtype == torch.int8:
        return SA_I8
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda or not t.is_contiguous():
        raise ValueError("tensors passed to the library must be contiguous device tensors")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


@dataclass
class KVCache:
    """Caller-owned paged K/V of one layer."""
    k: torch.Tensor
    v: torch.Tensor
    k_scale: Optional[torch.Tensor] = None  # int16/uint16-viewed fp16 bits or torch.float16 [P,16,Hkv]
    v_scale: Optional[torch.Tensor] = None

    def struct(self) -> sa_kv_cache:
        P, S, Hkv, d = self.k.shape
        return sa_kv_cache(_ptr(self.k), _ptr(self.v), _ptr(self.k_scale), _ptr(self.v_scale),
                           _dtype_code(self.k), P, S, Hkv, d)


@dataclass
class Seqs:
    page_table: torch.Tensor  # int32 [B, max_pages]
    seq_lens: torch.Tensor    # int32 [B]

    def struct(self) -> sa_seqs:
        B, mp = self.page_table.shape
        return sa_seqs(_ptr(self.page_table), _ptr(self.seq_lens), B, mp)


@dataclass
class SelectCfg:
    mode: int = SA_MODE_QUEST
    unit_tokens: int = 16
    k_compete: int = 14
    n_head_forced: int = 1
    n_tail_forced: int = 1
    rank: int = 16
    proj: Optional[torch.Tensor] = None  # fp32 [128, rank] (SALS)
    lse_scale: float = 0.0
    n_probe: int = 8                      # keys probed per block (PROBE)
    per_head: int = 0                     # QUEST: one selection per query head

    def struct(self) -> sa_select_cfg:
        return sa_select_cfg(self.mode, self.unit_tokens, self.k_compete, self.n_head_forced,
                             self.n_tail_forced, self.rank, _ptr(self.proj), self.lse_scale,
                             self.n_probe, self.per_head)


# ---------------------------------------------------------------- sizes
def sa_meta_bytes(kv: KVCache, cfg: SelectCfg) -> int:
    return load().sa_meta_bytes(ctypes.byref(kv.struct()), ctypes.byref(cfg.struct()))


def sa_meta_scale_bytes(kv: KVCache, cfg: SelectCfg) -> int:
    return load().sa_meta_scale_bytes(ctypes.byref(kv.struct()), ctypes.byref(cfg.struct()))


def sa_max_units(seqs: Seqs, cfg: SelectCfg) -> int:
    return load().sa_max_units(ctypes.byref(seqs.struct()), ctypes.byref(cfg.struct()))


def sa_max_selected(seqs: Seqs, cfg: SelectCfg) -> int:
    return load().sa_max_selected(ctypes.byref(seqs.struct()), ctypes.byref(cfg.struct()))


def sa_attn_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_pages: int,
                           max_sel: int) -> int:
    return load().sa_attn_workspace_size(batch, num_q_heads, num_kv_heads, max_pages, max_sel)


def sa_attn_heads_workspace_size(batch: int, num_q_heads: int, num_kv_heads: int, max_pages: int,
                                 max_sel: int) -> int:
    return load().sa_attn_heads_workspace_size(batch, num_q_heads, num_kv_heads, max_pages, max_sel)


def sa_decode_step_workspace_size(num_q_heads: int, kv: KVCache, seqs: Seqs, cfg: SelectCfg) -> int:
    return load().sa_decode_step_workspace_size(num_q_heads, ctypes.byref(kv.struct()),
                                                ctypes.byref(seqs.struct()),
                                                ctypes.byref(cfg.struct()))


def alloc_meta(kv: KVCache, cfg: SelectCfg):
    """Device buffers for sa_build_page_meta: (meta, meta_scale or None)."""
    dev = kv.k.device
    P, S, Hkv, d = kv.k.shape
    if cfg.mode == SA_MODE_PROBE:  # scores read K itself: no metadata
        return None, None
    if cfg.mode == SA_MODE_QUEST:
        return torch.empty((Hkv, P, 2, d), dtype=kv.k.dtype, device=dev), None
    return (torch.empty((P, S, Hkv, cfg.rank // 2), dtype=torch.uint8, device=dev),
            torch.empty((P, S, Hkv), dtype=torch.int16, device=dev))


def alloc_workspace(nbytes: int, device) -> torch.Tensor:
    """Zero-filled device workspace (sa_decode_step needs its hand-off words zero on first use)."""
    return torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)


# ---------------------------------------------------------------- entry points
def sa_build_page_meta(kv: KVCache, seqs: Seqs, cfg: SelectCfg, meta: torch.Tensor,
                       meta_scale: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(load().sa_build_page_meta(ctypes.byref(kv.struct()), ctypes.byref(seqs.struct()),
                                     ctypes.byref(cfg.struct()), _ptr(meta), _ptr(meta_scale),
                                     _stream(stream)), "sa_build_page_meta")


def sa_append_kv(k_new: torch.Tensor, v_new: torch.Tensor, kv: KVCache, seqs: Seqs, cfg: SelectCfg,
                 meta: torch.Tensor, meta_scale: Optional[torch.Tensor] = None,
                 k_scale_new: Optional[torch.Tensor] = None, v_scale_new: Optional[torch.Tensor] = None,
                 stream=None) -> None:
    """Writes one new token per sequence (at seq_lens[b] - 1) into kv and updates meta."""
    _check(load().sa_append_kv(_ptr(k_new), _ptr(v_new), _ptr(k_scale_new), _ptr(v_scale_new),
                               ctypes.byref(kv.struct()), ctypes.byref(seqs.struct()),
                               ctypes.byref(cfg.struct()), _ptr(meta), _ptr(meta_scale),
                               _stream(stream)), "sa_append_kv")


def sa_score_pages(q: torch.Tensor, kv: KVCache, seqs: Seqs, cfg: SelectCfg, meta: torch.Tensor,
                   meta_scale: Optional[torch.Tensor], scores: torch.Tensor, stream=None) -> None:
    _check(load().sa_score_pages(_ptr(q), _dtype_code(q), q.shape[1], ctypes.byref(kv.struct()),
                                 ctypes.byref(seqs.struct()), ctypes.byref(cfg.struct()),
                                 _ptr(meta), _ptr(meta_scale), _ptr(scores), _stream(stream)),
           "sa_score_pages")


def sa_topk_pages(scores: torch.Tensor, num_kv_heads: int, seqs: Seqs, cfg: SelectCfg,
                  sel: torch.Tensor, num_sel: torch.Tensor, stream=None) -> None:
    _check(load().sa_topk_pages(_ptr(scores), num_kv_heads, ctypes.byref(seqs.struct()),
                                ctypes.byref(cfg.struct()), _ptr(sel), _ptr(num_sel),
                                _stream(stream)), "sa_topk_pages")


def sa_sparse_decode_attn(q: torch.Tensor, kv: KVCache, seqs: Seqs, sel: Optional[torch.Tensor],
                          num_sel: Optional[torch.Tensor], softmax_scale: float, out: torch.Tensor,
                          workspace: torch.Tensor, stream=None) -> None:
    max_sel = 0 if sel is None else sel.shape[-1]
    _check(load().sa_sparse_decode_attn(_ptr(q), _dtype_code(q), q.shape[1],
                                        ctypes.byref(kv.struct()), ctypes.byref(seqs.struct()),
                                        _ptr(sel), _ptr(num_sel), max_sel, softmax_scale,
                                        _ptr(out), _ptr(workspace), workspace.numel(),
                                        _stream(stream)), "sa_sparse_decode_attn")


def sa_sparse_decode_attn_noalloc(q: torch.Tensor, kv: KVCache, seqs: Seqs,
                                  sel: Optional[torch.Tensor], num_sel: Optional[torch.Tensor],
                                  softmax_scale: float, out: torch.Tensor, stream=None) -> None:
    """sa_sparse_decode_attn with the library's own per-GPU scratch instead of a workspace."""
    max_sel = 0 if sel is None else sel.shape[-1]
    _check(load().sa_sparse_decode_attn_noalloc(_ptr(q), _dtype_code(q), q.shape[1],
                                                ctypes.byref(kv.struct()), ctypes.byref(seqs.struct()),
                                                _ptr(sel), _ptr(num_sel), max_sel, softmax_scale,
                                                _ptr(out), _stream(stream)),
           "sa_sparse_decode_attn_noalloc")


def sa_sparse_decode_attn_heads(q: torch.Tensor, kv: KVCache, seqs: Seqs, sel: torch.Tensor,
                                num_sel: torch.Tensor, softmax_scale: float, out: torch.Tensor,
                                workspace: torch.Tensor, stream=None) -> None:
    """Attention with one page list per query head (sel [B, Hq, max_sel])."""
    _check(load().sa_sparse_decode_attn_heads(_ptr(q), _dtype_code(q), q.shape[1],
                                              ctypes.byref(kv.struct()), ctypes.byref(seqs.struct()),
                                              _ptr(sel), _ptr(num_sel), sel.shape[-1], softmax_scale,
                                              _ptr(out), _ptr(workspace), workspace.numel(),
                                              _stream(stream)), "sa_sparse_decode_attn_heads")


def sa_decode_step(q: torch.Tensor, kv: KVCache, seqs: Seqs, cfg: SelectCfg, meta: torch.Tensor,
                   meta_scale: Optional[torch.Tensor], softmax_scale: float, out: torch.Tensor,
                   workspace: torch.Tensor, sel: Optional[torch.Tensor] = None,
                   num_sel: Optional[torch.Tensor] = None, stream=None) -> None:
    _check(load().sa_decode_step(_ptr(q), _dtype_code(q), q.shape[1], ctypes.byref(kv.struct()),
                                 ctypes.byref(seqs.struct()), ctypes.byref(cfg.struct()),
                                 _ptr(meta), _ptr(meta_scale), softmax_scale, _ptr(out),
                                 _ptr(sel), _ptr(num_sel), _ptr(workspace), workspace.numel(),
                                 _stream(stream)), "sa_decode_step")


def sa_stream_read(src: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Measurement helper: one streaming read of every byte of src (see include/sa.h)."""
    _check(load().sa_stream_read(_ptr(src), src.numel() * src.element_size(), _ptr(sink),
                                 sink.numel(), _stream(stream)), "sa_stream_read")
