"""Seeded synthetic workloads for query-aware sparse decode attention.

This package only generates inputs (and states how many bytes a decode step
must move); it holds none of the scoring, selection or attention arithmetic.
The CPU oracle and the GPU library both consume the arrays it returns.

Workloads follow the shapes and value distributions of the pages' settings:
a Llama-7B-like layer at 32K (Quest explainer, "background" KV-size
arithmetic and the kernel-level evaluation at 32K with a 2048-token budget),
passkey-style planted needles (Quest explainer, passkey retrieval table),
GQA models with int8 KV and an int4 low-rank index key (SALS on Ascend,
QSI and SFAA sections), and 16-token pages (Quest explainer, page-level
management section).  No public benchmark items are used.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA_SYNTH_LIB: load another build of synth.c (the sanitizer test's instrumented copy)
_LIB_PATH = os.environ.get("SA_SYNTH_LIB") or os.path.join(_HERE, "libsynth.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
_lib = None

PAGE = 16
HEAD_DIM = 128

# tensor ids of the counter-based streams
T_Q, T_K, T_V, T_QSCALE, T_KSCALE, T_VSCALE = 1, 2, 3, 4, 5, 6
T_NEEDLE_PAGE, T_NEEDLE_SLOT, T_LENS, T_PERM, T_OUTLIER, T_PROJ = 7, 8, 9, 10, 11, 12
T_FRESH_Q = 1000  # + step index


def build(verbose: bool = False, out: Optional[str] = None, sanitize: bool = False) -> str:
    """Compile synth.c into libsynth.so (gcc, OpenMP, no FP contraction); sanitize: an
    AddressSanitizer + UndefinedBehaviorSanitizer build (written to out)."""
    src = os.path.join(_HERE, "synth.c")
    dst = out or _LIB_PATH
    tmp = dst + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", *(SANITIZE_FLAGS if sanitize else []), "-o", tmp, src, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.check_call(cmd)
    os.replace(tmp, dst)
    return dst


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    u64, i64, dbl, vp = ctypes.c_uint64, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
    lib.synth_normal.argtypes = [u64, u64, u64, u64, dbl, dbl, vp, u64, ctypes.c_int, vp]
    lib.synth_uniform.argtypes = [u64, u64, u64, dbl, dbl, vp]
    lib.synth_uniform_int.argtypes = [u64, u64, u64, i64, i64, vp]
    lib.synth_permutation.argtypes = [u64, u64, u64, vp]
    lib.synth_quant_int8_rows.argtypes = [vp, u64, ctypes.c_int32, vp, vp]
    lib.synth_f32_to_bf16.argtypes = [vp, u64, vp]
    lib.synth_f32_to_f16.argtypes = [vp, u64, vp]
    lib.synth_f16_to_f32.argtypes = [vp, u64, vp]
    for f in (lib.synth_normal, lib.synth_uniform, lib.synth_uniform_int, lib.synth_permutation,
              lib.synth_quant_int8_rows, lib.synth_f32_to_bf16, lib.synth_f32_to_f16,
              lib.synth_f16_to_f32):
        f.restype = None
    _lib = lib
    return lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


# ----------------------------------------------------------------------------
# primitive streams
# ----------------------------------------------------------------------------
def normal(seed: int, tid: int, shape, dtype: str = "f32", mean: float = 0.0, std: float = 1.0,
           chan_scale: Optional[np.ndarray] = None, offset: int = 0) -> np.ndarray:
    """N(mean, std^2) values of stream (seed, tid); 'bf16' returns uint16 bits."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32 if dtype == "f32" else np.uint16)
    cs = None
    if chan_scale is not None:
        cs = np.ascontiguousarray(chan_scale, dtype=np.float32).ravel()
    _load().synth_normal(seed, tid, offset, n, mean, std, _ptr(cs), 0 if cs is None else cs.size,
                         0 if dtype == "f32" else 1, _ptr(out))
    return out.reshape(shape)


def uniform(seed: int, tid: int, n: int, lo: float, hi: float) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)
    _load().synth_uniform(seed, tid, n, lo, hi, _ptr(out))
    return out


def uniform_int(seed: int, tid: int, n: int, lo: int, hi: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_uniform_int(seed, tid, n, lo, hi, _ptr(out))
    return out


def permutation(seed: int, tid: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().synth_permutation(seed, tid, n, _ptr(out))
    return out


def quant_int8_rows(x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row symmetric int8 codes and fp16 scale bits (the caller-side KV format)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    row_len = x.shape[-1]
    rows = x.size // row_len
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[:-1], dtype=np.uint16)
    _load().synth_quant_int8_rows(_ptr(x), rows, row_len, _ptr(codes), _ptr(scales))
    return codes, scales


def f32_to_bf16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_f32_to_bf16(_ptr(x), x.size, _ptr(out))
    return out


def f32_to_f16(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _load().synth_f32_to_f16(_ptr(x), x.size, _ptr(out))
    return out


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Widen bf16 bits to float32 (exact)."""
    return (np.ascontiguousarray(x, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def f16_to_f32(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.uint16)
    out = np.empty(x.shape, dtype=np.float32)
    _load().synth_f16_to_f32(_ptr(x), x.size, _ptr(out))
    return out


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    d: int
    kv_dtype: str          # 'f32' | 'bf16' | 'i8'
    q_dtype: str           # 'f32' | 'bf16'
    q: np.ndarray          # [B, Hq, d] float32 or bf16 bits
    k: np.ndarray          # [P, 16, Hkv, d]
    v: np.ndarray
    k_scale: Optional[np.ndarray]  # fp16 bits [P, 16, Hkv] (int8 KV only)
    v_scale: Optional[np.ndarray]
    page_table: np.ndarray  # int32 [B, max_pages]; -1 past each sequence's pages
    seq_lens: np.ndarray    # int32 [B]
    mode: str               # 'quest' | 'sals' | 'probe'
    unit_tokens: int
    k_compete: int
    n_head_forced: int
    n_tail_forced: int
    proj: Optional[np.ndarray] = None  # float32 [d, rank] (SALS)
    rank: int = 16
    lse_scale: float = 0.0
    softmax_scale: float = 0.0
    seed: int = 0
    needles: List[Tuple[int, int, int, int]] = field(default_factory=list)  # (b, kv_head, page, slot)
    n_probe: int = 8        # probe sampling: keys probed per block

    @property
    def num_pages(self) -> int:
        return int(self.k.shape[0])

    @property
    def max_pages(self) -> int:
        return int(self.page_table.shape[1])

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def unit_pages(self) -> int:
        return self.unit_tokens // PAGE

    def n_pages(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // PAGE)

    def n_units(self, b: int) -> int:
        return -(-int(self.seq_lens[b]) // self.unit_tokens)

    @property
    def max_units(self) -> int:
        return -(-self.max_pages // self.unit_pages)

    @property
    def max_sel(self) -> int:
        return min((self.k_compete + self.n_head_forced + self.n_tail_forced) * self.unit_pages,
                   self.max_pages)


def _elt(dtype: str) -> int:
    return {"f32": 4, "bf16": 2, "i8": 1}[dtype]


def fresh_q(wl: Workload, step: int) -> np.ndarray:
    """A new seeded query of the workload's shape (one per timed decode step)."""
    return normal(wl.seed, T_FRESH_Q + step, (wl.B, wl.Hq, wl.d), wl.q_dtype)


def _q_to_f64(wl: Workload, q: np.ndarray) -> np.ndarray:
    return (bf16_to_f32(q) if wl.q_dtype == "bf16" else q).astype(np.float64)


def _plant_needles(wl: Workload, pages: np.ndarray, slots: np.ndarray, heads: np.ndarray,
                   batches: np.ndarray, alpha: float = 4.0) -> None:
    """Overwrite key (b, h, page, slot) with alpha * q/|q| of the matching query head."""
    qd = _q_to_f64(wl, wl.q)
    for b, h, p, s in zip(batches, heads, pages, slots):
        b, h, p, s = int(b), int(h), int(p), int(s)
        qh = qd[b, h * wl.G]  # needles are planted for MHA workloads (G == 1)
        key = alpha * qh / np.linalg.norm(qh)
        pp = int(wl.page_table[b, p])
        if wl.kv_dtype == "f32":
            wl.k[pp, s, h, :] = key.astype(np.float32)
        elif wl.kv_dtype == "bf16":
            wl.k[pp, s, h, :] = f32_to_bf16(key.astype(np.float32))
        else:
            raise ValueError("needles are planted only in f32/bf16 caches")
        wl.needles.append((b, h, p, s))


def contiguous_page_table(lens: np.ndarray, max_pages: int) -> Tuple[np.ndarray, int]:
    B = len(lens)
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    nxt = 0
    for b in range(B):
        n = -(-int(lens[b]) // PAGE)
        pt[b, :n] = np.arange(nxt, nxt + n, dtype=np.int32)
        nxt += n
    return pt, nxt


def random_page_table(seed: int, lens: np.ndarray, max_pages: int) -> Tuple[np.ndarray, int]:
    """Each sequence's pages are drawn from one shuffled physical pool."""
    B = len(lens)
    ns = [-(-int(L) // PAGE) for L in lens]
    pool = permutation(seed, T_PERM, sum(ns))
    pt = np.full((B, max_pages), -1, dtype=np.int32)
    o = 0
    for b in range(B):
        pt[b, :ns[b]] = pool[o:o + ns[b]]
        o += ns[b]
    return pt, sum(ns)


def make_custom(B: int = 1, Hq: int = 8, Hkv: int = 8, lens=(2048,), kv_dtype: str = "bf16",
                q_dtype: str = "bf16", mode: str = "quest", budget_pages: Optional[int] = None,
                k_compete: Optional[int] = None, n_head_forced: Optional[int] = None,
                n_tail_forced: Optional[int] = None, unit_tokens: Optional[int] = None,
                page_table: str = "contiguous", seed: int = 7, max_pages: Optional[int] = None,
                kv_chan_scale: Optional[np.ndarray] = None, q_chan_scale: Optional[np.ndarray] = None,
                rank: int = 16, extra_pages: int = 0, name: str = "custom",
                n_probe: int = 8) -> Workload:
    """Seeded workload of arbitrary shape (used for parity cases and config builders).

    kv_dtype 'i8' draws fp32 N(0,1) keys/values and quantises each
    (token, kv-head) row symmetrically (scale = amax/127 stored fp16)."""
    d = HEAD_DIM
    lens = np.asarray(lens, dtype=np.int32)
    assert len(lens) == B
    mp = max_pages if max_pages is not None else max(1, -(-int(lens.max()) // PAGE))
    if page_table == "contiguous":
        pt, P = contiguous_page_table(lens, mp)
    else:
        pt, P = random_page_table(seed, lens, mp)
    P = max(P + extra_pages, 1)
    q = normal(seed, T_Q, (B, Hq, d), q_dtype, chan_scale=q_chan_scale)
    if kv_dtype == "i8":
        kf = normal(seed, T_K, (P, PAGE, Hkv, d), "f32", chan_scale=kv_chan_scale)
        k, ks = quant_int8_rows(kf)
        del kf
        vf = normal(seed, T_V, (P, PAGE, Hkv, d), "f32", chan_scale=kv_chan_scale)
        v, vs = quant_int8_rows(vf)
        del vf
    else:
        k = normal(seed, T_K, (P, PAGE, Hkv, d), kv_dtype, chan_scale=kv_chan_scale)
        v = normal(seed, T_V, (P, PAGE, Hkv, d), kv_dtype, chan_scale=kv_chan_scale)
        ks = vs = None
    if mode == "quest":
        ut = unit_tokens or PAGE
        fh = 1 if n_head_forced is None else n_head_forced
        ft = 1 if n_tail_forced is None else n_tail_forced
        if k_compete is None:
            k_compete = (budget_pages if budget_pages is not None else 16) - fh - ft
        proj = None
    elif mode == "probe":
        ut = unit_tokens or 32
        fh = 0 if n_head_forced is None else n_head_forced
        ft = 1 if n_tail_forced is None else n_tail_forced
        if k_compete is None:
            k_compete = (budget_pages * PAGE // ut if budget_pages is not None else 32) - fh - ft
        proj = None
    else:
        ut = unit_tokens or 64
        fh = 0 if n_head_forced is None else n_head_forced
        ft = 2 if n_tail_forced is None else n_tail_forced
        if k_compete is None:
            k_compete = 32
        proj = normal(seed, T_PROJ, (d, rank), "f32", std=1.0 / math.sqrt(rank))
    return Workload(name=name, B=B, Hq=Hq, Hkv=Hkv, d=d, kv_dtype=kv_dtype, q_dtype=q_dtype, q=q,
                    k=k, v=v, k_scale=ks, v_scale=vs, page_table=pt, seq_lens=lens, mode=mode,
                    unit_tokens=ut, k_compete=int(k_compete), n_head_forced=fh, n_tail_forced=ft,
                    proj=proj, rank=rank, lse_scale=1.0 / math.sqrt(d),
                    softmax_scale=1.0 / math.sqrt(d), seed=seed, n_probe=n_probe)


CONFIG_NAMES = {
    1: "tiny MHA decode: B=1 Hq=Hkv=8 d=128 L=2048 fp32, budget 16 pages",
    2: "Llama-7B-like layer decode: B=1 Hq=Hkv=32 d=128 L=32768 bf16, budget 2048 tokens",
    3: "GQA batched decode: B=16 Hq=32 Hkv=8 d=128 L~U[8192,32768] bf16, budget 4096 tokens",
    4: "SALS int4 index + int8 KV: B=4 Hq=32 Hkv=8 d=128 L=131072, top-32 blocks + 2 tail",
    5: "large decode batch: B=8 Hq=64 Hkv=8 d=128 L=262144 bf16, budget 4096 tokens",
}


def make_config(cfg: int, layer_copy: int = 0, dense: bool = False, probe: bool = False) -> Workload:
    """The five reference workloads at full size.  seed = 1000*cfg + layer_copy.
    probe: the same inputs selected by probe sampling instead (32-token blocks, 8 probes,
    the same token budget: budget/32 - 1 blocks by score plus the last block)."""
    seed = 1000 * cfg + layer_copy
    d = HEAD_DIM
    if cfg == 1:
        wl = make_custom(B=1, Hq=8, Hkv=8, lens=(2048,), kv_dtype="f32", q_dtype="f32",
                         budget_pages=16, seed=seed, name="cfg1")
        n = wl.n_pages(0)
        heads = np.arange(8)
        pages = uniform_int(seed, T_NEEDLE_PAGE, 8, 1, n - 2)
        slots = uniform_int(seed, T_NEEDLE_SLOT, 8, 0, PAGE - 1)
        _plant_needles(wl, pages, slots, heads, np.zeros(8, dtype=np.int32))
    elif cfg == 2:
        H = 32
        qs = uniform(seed, T_QSCALE, H * d, 0.5, 2.0)
        kvs_k = uniform(seed, T_KSCALE, H * d, 0.5, 2.0)
        kvs_v = uniform(seed, T_VSCALE, H * d, 0.5, 2.0)
        L = 32768
        lens = np.array([L], dtype=np.int32)
        pt, P = contiguous_page_table(lens, L // PAGE)
        q = normal(seed, T_Q, (1, H, d), "bf16", chan_scale=qs)
        k = normal(seed, T_K, (P, PAGE, H, d), "bf16", chan_scale=kvs_k)
        v = normal(seed, T_V, (P, PAGE, H, d), "bf16", chan_scale=kvs_v)
        wl = Workload(name="cfg2", B=1, Hq=H, Hkv=H, d=d, kv_dtype="bf16", q_dtype="bf16", q=q,
                      k=k, v=v, k_scale=None, v_scale=None, page_table=pt, seq_lens=lens,
                      mode="quest", unit_tokens=PAGE, k_compete=128 - 2, n_head_forced=1,
                      n_tail_forced=1, lse_scale=1 / math.sqrt(d), softmax_scale=1 / math.sqrt(d),
                      seed=seed)
        n = L // PAGE
        for h in range(H):
            # 8 needles per head at distinct pages of the non-forced range [1, n-2]
            perm = permutation(seed, T_NEEDLE_PAGE * 100 + h, n - 2)[:8] + 1
            slots = uniform_int(seed, T_NEEDLE_SLOT * 100 + h, 8, 0, PAGE - 1)
            _plant_needles(wl, perm, slots, np.full(8, h), np.zeros(8, dtype=np.int32))
    elif cfg == 3:
        B, Hq, Hkv = 16, 32, 8
        lens = uniform_int(seed, T_LENS, B, 8192, 32768)
        n_out = math.ceil(0.01 * Hkv * d)
        chans = permutation(seed, T_OUTLIER, Hkv * d)[:n_out]
        cs = np.ones(Hkv * d, dtype=np.float32)
        cs[chans] = 8.0
        wl = make_custom(B=B, Hq=Hq, Hkv=Hkv, lens=lens, kv_dtype="bf16", q_dtype="bf16",
                         budget_pages=4096 // PAGE, page_table="random", seed=seed,
                         max_pages=32768 // PAGE, kv_chan_scale=cs, name="cfg3")
    elif cfg == 4:
        wl = make_custom(B=4, Hq=32, Hkv=8, lens=(131072,) * 4, kv_dtype="i8", q_dtype="bf16",
                         mode="sals", k_compete=2048 // 64, n_head_forced=0, n_tail_forced=2,
                         unit_tokens=64, seed=seed, name="cfg4")
    elif cfg == 5:
        wl = make_custom(B=8, Hq=64, Hkv=8, lens=(262144,) * 8, kv_dtype="bf16", q_dtype="bf16",
                         budget_pages=4096 // PAGE, seed=seed, name="cfg5")
    else:
        raise ValueError(cfg)
    if probe:
        budget = (wl.k_compete + wl.n_head_forced + wl.n_tail_forced) * wl.unit_tokens
        wl.mode, wl.unit_tokens, wl.n_probe = "probe", 32, 8
        wl.n_head_forced, wl.n_tail_forced = 0, 1
        wl.k_compete = budget // 32 - 1
        wl.proj = None
        wl.name += "-probe"
    if dense:
        wl.k_compete = wl.max_units
        wl.name += "-dense"
    return wl


# ----------------------------------------------------------------------------
# bytes model
# ----------------------------------------------------------------------------
def kv_cache_bytes(n_layer: int, L: int, n_kv_head: int, d_head: int, elt: int = 2) -> int:
    """K and V of every layer: 2 * N_layer * L * n_head * d_head * elt (Quest explainer, background)."""
    return 2 * n_layer * L * n_kv_head * d_head * elt


def quest_read_ratio(page_size: int, L: int, k_pages: int) -> float:
    """Metadata read plus top-K pages read, over the full KV read: 1/S + K*S/L
    (Quest explainer, read-volume formula of the three-kernel pipeline)."""
    return 1.0 / page_size + k_pages * page_size / L


def step_bytes(wl: Workload, num_sel: Optional[np.ndarray] = None) -> dict:
    """Algorithmic HBM bytes of one decode step (scoring + selection + attention).

    meta    : Quest min/max metadata of every page of every sequence (2*d values in the
              KV dtype per page and kv-head), or the SALS index key of every token
              (rank/2 code bytes + 2 scale bytes per token and kv-head, whole pages), or the
              probed key rows of every block (probe sampling);
    kv      : K and V of the selected pages (16 tokens each), plus int8 scales;
    q / out : the query (q dtype) and the fp32 output.
    Score and partial-result traffic is not counted."""
    e = _elt(wl.kv_dtype)
    npages = np.array([wl.n_pages(b) for b in range(wl.B)], dtype=np.int64)
    if wl.mode == "quest":
        meta = int(npages.sum()) * wl.Hkv * 2 * wl.d * e
    elif wl.mode == "probe":  # the probed key rows of every block (n_probe per full block)
        meta = 0
        for b in range(wl.B):
            L = int(wl.seq_lens[b])
            for t0 in range(0, L, wl.unit_tokens):
                n = min(wl.unit_tokens, L - t0)
                step = max(1, n // wl.n_probe)
                meta += -(-n // step) * wl.Hkv * wl.d * e
    else:
        meta = int(npages.sum()) * PAGE * wl.Hkv * (wl.rank // 2 + 2)
    if num_sel is None:
        nsel = np.array([[min(wl.n_pages(b), wl.max_sel) for _ in range(wl.Hkv)]
                         for b in range(wl.B)], dtype=np.int64)
    else:
        nsel = np.asarray(num_sel, dtype=np.int64)
    per_page = PAGE * wl.d * e * 2 + (PAGE * 2 * 2 if wl.kv_dtype == "i8" else 0)
    kv = int(nsel.sum()) * per_page
    qb = wl.B * wl.Hq * wl.d * _elt(wl.q_dtype)
    ob = wl.B * wl.Hq * wl.d * 4
    return {"meta": meta, "kv": kv, "q": qb, "out": ob, "total": meta + kv + qb + ob}


def dense_bytes(wl: Workload) -> int:
    """Bytes of dense decode attention over every valid page: all K/V + q + out."""
    e = _elt(wl.kv_dtype)
    npages = sum(wl.n_pages(b) for b in range(wl.B))
    per_page = PAGE * wl.d * e * 2 + (PAGE * 2 * 2 if wl.kv_dtype == "i8" else 0)
    return npages * wl.Hkv * per_page + wl.B * wl.Hq * wl.d * (_elt(wl.q_dtype) + 4)


# ----------------------------------------------------------------------------
# device copies (torch used only as an allocator)
# ----------------------------------------------------------------------------
def _to_torch(a: Optional[np.ndarray], kind: str, device):
    import torch
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    elif kind == "f16bits":
        t = torch.from_numpy(a.view(np.int16))
    else:
        t = torch.from_numpy(a)
    return t.to(device, non_blocking=False)


@dataclass
class DeviceWorkload:
    q: object
    k: object
    v: object
    k_scale: object
    v_scale: object
    page_table: object
    seq_lens: object
    proj: object


def to_device(wl: Workload, device="cuda", q: Optional[np.ndarray] = None) -> DeviceWorkload:
    """Copy a workload's arrays to device tensors of matching dtypes (bf16 bits -> torch.bfloat16,
    fp16 scale bits -> torch.int16)."""
    q = wl.q if q is None else q
    kvk = "bf16" if wl.kv_dtype == "bf16" else "raw"
    return DeviceWorkload(
        q=_to_torch(q, "bf16" if wl.q_dtype == "bf16" else "raw", device),
        k=_to_torch(wl.k, kvk, device), v=_to_torch(wl.v, kvk, device),
        k_scale=_to_torch(wl.k_scale, "f16bits", device),
        v_scale=_to_torch(wl.v_scale, "f16bits", device),
        page_table=_to_torch(wl.page_table, "raw", device),
        seq_lens=_to_torch(wl.seq_lens, "raw", device),
        proj=_to_torch(wl.proj, "raw", device))


def q_to_device(wl: Workload, q: np.ndarray, device="cuda"):
    return _to_torch(q, "bf16" if wl.q_dtype == "bf16" else "raw", device)
