"""CPU oracle of query-aware sparse decode attention (numpy front end).

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg are the only users.  The product path never imports this
package.  The arithmetic lives in sa_oracle.c (plain C, double accumulation),
which shares no code with the GPU library; this module only marshals numpy
arrays and composes the oracle's steps in the order the pages give them:
score every unit, select an exact top-K with forced sink/tail units, attend
over the selected pages.

Parity pins: every function here is pinned by tests/test_oracle_*.py against
closed forms, invariants, brute force or independent library routines.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# SA_ORACLE_LIB: load another build of sa_oracle.c (the sanitizer test's instrumented copy)
_LIB_PATH = os.environ.get("SA_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
SANITIZE_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
_lib = None

DTYPES = {"f32": 0, "bf16": 1, "i8": 2}
PAGE = 16


def build(verbose: bool = False, out: Optional[str] = None, sanitize: bool = False) -> str:
    """Compile sa_oracle.c into liboracle.so; sanitize: an AddressSanitizer +
    UndefinedBehaviorSanitizer build (written to out)."""
    src = os.path.join(_HERE, "sa_oracle.c")
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
    i, d, vp = ctypes.c_int, ctypes.c_double, ctypes.c_void_p
    lib.oracle_quest_meta.argtypes = [vp, i, i, i, i, i, vp, vp, i, i, vp]
    lib.oracle_quest_meta.restype = i
    lib.oracle_quest_scores.argtypes = [vp, i, i, vp, i, i, i, i, i, vp, vp, i, i, vp, vp]
    lib.oracle_quest_scores.restype = None
    lib.oracle_sals_index.argtypes = [vp, i, vp, i, i, i, i, vp, vp, i, i, vp, i, vp, vp]
    lib.oracle_sals_index.restype = i
    lib.oracle_sals_scores.argtypes = [vp, i, i, vp, vp, i, i, i, vp, i, vp, vp, i, i, i, d, vp, vp]
    lib.oracle_sals_scores.restype = None
    lib.oracle_sals_scores_float.argtypes = [vp, i, i, vp, i, i, i, vp, i, vp, vp, i, i, i, d, vp]
    lib.oracle_sals_scores_float.restype = None
    lib.oracle_select.argtypes = [vp, i, i, i, vp, i, i, i, i, i, i, vp, vp]
    lib.oracle_select.restype = i
    lib.oracle_probe_scores.argtypes = [vp, i, i, vp, i, vp, i, i, i, vp, vp, i, i, i, i, vp, vp]
    lib.oracle_probe_scores.restype = None
    lib.oracle_attention.argtypes = [vp, i, i, vp, vp, i, vp, vp, i, i, i, vp, vp, i, i, vp, vp, i,
                                     d, vp, i, vp]
    lib.oracle_attention.restype = None
    lib.oracle_set_threads.argtypes = [i]
    lib.oracle_set_threads.restype = None
    lib.oracle_set_threads(1)  # single-threaded unless set_threads() says otherwise
    _lib = lib
    return lib


def set_threads(n: int) -> None:
    """Host threads of the oracle's outer loops (independent outputs; results do not depend
    on the count)."""
    _load().oracle_set_threads(int(n))


def _p(a: Optional[np.ndarray]):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype=None):
    return None if a is None else np.ascontiguousarray(a if dtype is None else a.astype(dtype, copy=False))


def quest_meta(k: np.ndarray, kv_dtype: str, page_table: np.ndarray, seq_lens: np.ndarray,
               meta: Optional[np.ndarray] = None) -> np.ndarray:
    """Per (kv-head, page, dim) max (slot 0) and min (slot 1) over the page's valid tokens;
    layout [Hkv, P, 2, d]."""
    k = _c(k)
    P, S, Hkv, d = k.shape
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    if meta is None:
        meta = np.zeros((Hkv, P, 2, d), dtype=k.dtype)
    rc = _load().oracle_quest_meta(_p(k), DTYPES[kv_dtype], P, S, Hkv, d, _p(pt), _p(sl), pt.shape[0],
                                   pt.shape[1], _p(meta))
    if rc != 0:
        raise ValueError(f"oracle_quest_meta failed ({rc})")
    return meta


def quest_scores(q: np.ndarray, q_dtype: str, meta: np.ndarray, kv_dtype: str,
                 page_table: np.ndarray, seq_lens: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Group score max_g sum_i max(q_gi m_i, q_gi M_i) per (b, kv-head, page), plus its
    absolute magnitude; pages past the sequence get -inf."""
    q, meta = _c(q), _c(meta)
    B, Hq, d = q.shape
    Hkv, P = meta.shape[0], meta.shape[1]
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    mp = pt.shape[1]
    sc = np.empty((B, Hkv, mp), dtype=np.float64)
    ab = np.empty((B, Hkv, mp), dtype=np.float64)
    _load().oracle_quest_scores(_p(q), DTYPES[q_dtype], Hq, _p(meta), DTYPES[kv_dtype], Hkv, P, d,
                                PAGE, _p(pt), _p(sl), B, mp, _p(sc), _p(ab))
    return sc, ab


def sals_index(k: np.ndarray, kv_dtype: str, k_scale: Optional[np.ndarray], page_table: np.ndarray,
               seq_lens: np.ndarray, proj: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """int4 low-rank index key (codes [P,S,Hkv,rank/2] uint8, fp16 scale bits [P,S,Hkv])."""
    k = _c(k)
    P, S, Hkv, d = k.shape
    proj = _c(proj, np.float32)
    rank = proj.shape[1]
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    codes = np.zeros((P, S, Hkv, rank // 2), dtype=np.uint8)
    scales = np.zeros((P, S, Hkv), dtype=np.uint16)
    ks = _c(k_scale, np.uint16)
    rc = _load().oracle_sals_index(_p(k), DTYPES[kv_dtype], _p(ks), P, S, Hkv, d, _p(pt), _p(sl),
                                   pt.shape[0], pt.shape[1], _p(proj), rank, _p(codes), _p(scales))
    if rc != 0:
        raise ValueError(f"oracle_sals_index failed ({rc})")
    return codes, scales


def sals_scores(q: np.ndarray, q_dtype: str, codes: np.ndarray, scales: np.ndarray,
                proj: np.ndarray, page_table: np.ndarray, seq_lens: np.ndarray, num_kv_heads: int,
                unit_tokens: int, tau: float) -> Tuple[np.ndarray, np.ndarray]:
    """Block log-sum-exp of tau * (qbar P) . (scale * codes) per (b, kv-head, block)."""
    q, codes, scales = _c(q), _c(codes), _c(scales, np.uint16)
    B, Hq, d = q.shape
    proj = _c(proj, np.float32)
    rank = proj.shape[1]
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    mp = pt.shape[1]
    mu = -(-mp * PAGE // unit_tokens)
    sc = np.empty((B, num_kv_heads, mu), dtype=np.float64)
    ab = np.empty((B, num_kv_heads, mu), dtype=np.float64)
    _load().oracle_sals_scores(_p(q), DTYPES[q_dtype], Hq, _p(codes), _p(scales), num_kv_heads, PAGE,
                               rank, _p(proj), d, _p(pt), _p(sl), B, mp, unit_tokens, tau, _p(sc),
                               _p(ab))
    return sc, ab


def sals_scores_float(q: np.ndarray, q_dtype: str, keys_lr: np.ndarray, proj: np.ndarray,
                      page_table: np.ndarray, seq_lens: np.ndarray, unit_tokens: int,
                      tau: float) -> np.ndarray:
    """The SALS block scorer on unquantised low-rank keys [P, S, Hkv, rank] (fp32)."""
    q, keys_lr = _c(q), _c(keys_lr, np.float32)
    B, Hq, d = q.shape
    P, S, Hkv, rank = keys_lr.shape
    proj = _c(proj, np.float32)
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    mp = pt.shape[1]
    mu = -(-mp * PAGE // unit_tokens)
    sc = np.empty((B, Hkv, mu), dtype=np.float64)
    _load().oracle_sals_scores_float(_p(q), DTYPES[q_dtype], Hq, _p(keys_lr), Hkv, S, rank, _p(proj),
                                     d, _p(pt), _p(sl), B, mp, unit_tokens, tau, _p(sc))
    return sc


def probe_scores(q: np.ndarray, q_dtype: str, k: np.ndarray, kv_dtype: str,
                 k_scale: Optional[np.ndarray], page_table: np.ndarray, seq_lens: np.ndarray,
                 unit_tokens: int, n_probe: int) -> Tuple[np.ndarray, np.ndarray]:
    """Probe-sampling block scores: max over evenly probed tokens and the group's heads of
    q_g . k_t, plus the absolute magnitude; blocks past the sequence get -inf."""
    q, k = _c(q), _c(k)
    B, Hq, d = q.shape
    P, S, Hkv, _ = k.shape
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    mp = pt.shape[1]
    mu = -(-mp * PAGE // unit_tokens)
    sc = np.empty((B, Hkv, mu), dtype=np.float64)
    ab = np.empty((B, Hkv, mu), dtype=np.float64)
    _load().oracle_probe_scores(_p(q), DTYPES[q_dtype], Hq, _p(k), DTYPES[kv_dtype],
                                _p(_c(k_scale, np.uint16)), Hkv, S, d, _p(pt), _p(sl), B, mp,
                                unit_tokens, n_probe, _p(sc), _p(ab))
    return sc, ab


def select(scores: np.ndarray, seq_lens: np.ndarray, unit_tokens: int, k: int, n_head: int,
           n_tail: int, max_sel: int) -> Tuple[np.ndarray, np.ndarray]:
    """Exact top-k of the middle units + forced head/tail units, as ascending page lists."""
    scores = _c(scores, np.float64)
    B, Hkv, mu = scores.shape
    sl = _c(seq_lens, np.int32)
    sel = np.empty((B, Hkv, max_sel), dtype=np.int32)
    num = np.empty((B, Hkv), dtype=np.int32)
    rc = _load().oracle_select(_p(scores), B, Hkv, mu, _p(sl), PAGE, unit_tokens, k, n_head, n_tail,
                               max_sel, _p(sel), _p(num))
    if rc != 0:
        raise ValueError("selection exceeds max_sel")
    return sel, num


def attention(q: np.ndarray, q_dtype: str, k: np.ndarray, v: np.ndarray, kv_dtype: str,
              k_scale: Optional[np.ndarray], v_scale: Optional[np.ndarray],
              page_table: np.ndarray, seq_lens: np.ndarray, sel: Optional[np.ndarray],
              num_sel: Optional[np.ndarray], tau: float,
              rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Softmax attention over the selected pages (sel None: every page), fp32 output."""
    q, k, v = _c(q), _c(k), _c(v)
    B, Hq, d = q.shape
    P, S, Hkv, _ = k.shape
    pt, sl = _c(page_table, np.int32), _c(seq_lens, np.int32)
    sel_c = _c(sel, np.int32)
    num_c = _c(num_sel, np.int32)
    max_sel = 0 if sel_c is None else sel_c.shape[-1]
    rows_c = _c(rows, np.int32)
    nrows = 0 if rows_c is None else rows_c.size
    out = np.empty((nrows, d) if rows_c is not None else (B, Hq, d), dtype=np.float32)
    _load().oracle_attention(_p(q), DTYPES[q_dtype], Hq, _p(k), _p(v), DTYPES[kv_dtype],
                             _p(_c(k_scale, np.uint16)), _p(_c(v_scale, np.uint16)), Hkv, d, S,
                             _p(pt), _p(sl), B, pt.shape[1], _p(sel_c), _p(num_c), max_sel, tau,
                             _p(rows_c), nrows, _p(out))
    return out


# ----------------------------------------------------------------------------
# composed decode step (scores -> selection -> attention)
# ----------------------------------------------------------------------------
def quest_scores_per_head(q: np.ndarray, q_dtype: str, meta: np.ndarray, kv_dtype: str,
                          page_table: np.ndarray, seq_lens: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-head Quest selection scores ([Quest] GQA section: the per-head variant, each
    query head with its own pages): head h*G + g's own bound sum_i max(q_i m_i, q_i M_i)
    per page, i.e. the group score of a group of one, taken head slot g at a time.
    [B, Hq, max_pages] scores and magnitudes."""
    q = _c(q)
    B, Hq, d = q.shape
    G = Hq // meta.shape[0]
    mp = page_table.shape[1]
    sc = np.empty((B, Hq, mp), dtype=np.float64)
    ab = np.empty((B, Hq, mp), dtype=np.float64)
    for g in range(G):
        s, a = quest_scores(np.ascontiguousarray(q[:, g::G]), q_dtype, meta, kv_dtype, page_table,
                            seq_lens)
        sc[:, g::G], ab[:, g::G] = s, a
    return sc, ab


def attention_per_head(q: np.ndarray, q_dtype: str, k: np.ndarray, v: np.ndarray, kv_dtype: str,
                       k_scale: Optional[np.ndarray], v_scale: Optional[np.ndarray],
                       page_table: np.ndarray, seq_lens: np.ndarray, sel: np.ndarray,
                       num_sel: np.ndarray, tau: float) -> np.ndarray:
    """Each query head over its own pages: head h*G + g attends over sel[b, h*G + g]
    (the attention of a group of one, head slot g at a time).  [B, Hq, d] fp32."""
    q = _c(q)
    B, Hq, d = q.shape
    G = Hq // k.shape[2]
    out = np.empty((B, Hq, d), dtype=np.float32)
    for g in range(G):
        out[:, g::G] = attention(np.ascontiguousarray(q[:, g::G]), q_dtype, k, v, kv_dtype, k_scale,
                                 v_scale, page_table, seq_lens, np.ascontiguousarray(sel[:, g::G]),
                                 np.ascontiguousarray(num_sel[:, g::G]), tau)
    return out


def build_meta(wl) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Quest: (meta, None); SALS: (codes, scales); probe sampling: (None, None), it reads K."""
    if wl.mode == "probe":
        return None, None
    if wl.mode == "quest":
        return quest_meta(wl.k, wl.kv_dtype, wl.page_table, wl.seq_lens), None
    return sals_index(wl.k, wl.kv_dtype, wl.k_scale, wl.page_table, wl.seq_lens, wl.proj)


def score(wl, meta, meta_scale, q=None) -> Tuple[np.ndarray, np.ndarray]:
    q = wl.q if q is None else q
    if wl.mode == "probe":
        return probe_scores(q, wl.q_dtype, wl.k, wl.kv_dtype, wl.k_scale, wl.page_table,
                            wl.seq_lens, wl.unit_tokens, wl.n_probe)
    if wl.mode == "quest":
        return quest_scores(q, wl.q_dtype, meta, wl.kv_dtype, wl.page_table, wl.seq_lens)
    return sals_scores(q, wl.q_dtype, meta, meta_scale, wl.proj, wl.page_table, wl.seq_lens, wl.Hkv,
                       wl.unit_tokens, wl.lse_scale)


def decode_step(wl, meta, meta_scale, q=None, rows=None):
    """Oracle decode step: returns (out, sel, num_sel, scores, abs_scale)."""
    q = wl.q if q is None else q
    sc, ab = score(wl, meta, meta_scale, q)
    sel, num = select(sc, wl.seq_lens, wl.unit_tokens, wl.k_compete, wl.n_head_forced,
                      wl.n_tail_forced, wl.max_sel)
    out = attention(q, wl.q_dtype, wl.k, wl.v, wl.kv_dtype, wl.k_scale, wl.v_scale, wl.page_table,
                    wl.seq_lens, sel, num, wl.softmax_scale, rows=rows)
    return out, sel, num, sc, ab
