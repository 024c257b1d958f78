"""Pins of the oracle's SALS index key (int4 low-rank K*P) and block LSE scorer.

SALS on Ascend (QSI): the index query is the group-mean of q, the index key
is a low-rank int4-quantised key, and each block's score is a log-sum-exp of
its token scores (approximating the block's attention mass).  SequenceO1
explainer: the sketch key is K*P with a fixed random projection.
"""
import numpy as np
import pytest
import scipy.special

import oracle
import synth


def _decode_codes(codes):
    """Independent nibble decoder: low nibble = even index, two's complement."""
    lo = (codes & 0xF).astype(np.int32)
    hi = (codes >> 4).astype(np.int32)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(codes.shape[:-1] + (codes.shape[-1] * 2,), dtype=np.int32)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def test_index_with_one_hot_projection_is_exact_rounding():
    """P picks one key dimension per rank column, so kp_j = k_{pi(j)} exactly and the
    codes are rint(k / scale) with scale = fp16(amax / 7)."""
    wl = synth.make_custom(B=1, Hq=2, Hkv=2, lens=(40,), kv_dtype="f32", q_dtype="f32",
                           mode="sals", seed=3)
    pick = np.array([5, 0, 127, 64, 3, 9, 100, 77, 12, 13, 14, 15, 16, 88, 99, 1])
    P = np.zeros((128, 16), np.float32)
    P[pick, np.arange(16)] = 1.0
    codes, scales = oracle.sals_index(wl.k, "f32", None, wl.page_table, wl.seq_lens, P)
    c = _decode_codes(codes)
    for t in range(40):
        pp, s = wl.page_table[0, t // 16], t % 16
        for h in range(2):
            kp = wl.k[pp, s, h, pick]
            amax = np.float32(np.abs(kp).max())
            sc = (amax / np.float32(7.0)).astype(np.float16)
            assert scales[pp, s, h] == sc.view(np.uint16)
            want = np.clip(np.rint(kp / np.float32(sc)), -7, 7).astype(np.int32)
            assert np.array_equal(c[pp, s, h], want)
    # slots past the end of the sequence are zero
    assert not codes[wl.page_table[0, 2], 8:].any() and not scales[wl.page_table[0, 2], 8:].any()


def test_index_packing_low_nibble_first():
    k = np.zeros((1, 16, 1, 128), np.float32)
    k[0, 0, 0, :4] = [7.0, -7.0, 3.0, -1.0]
    P = np.zeros((128, 16), np.float32)
    P[np.arange(4), np.arange(4)] = 1.0
    pt = np.zeros((1, 1), np.int32)
    codes, scales = oracle.sals_index(k, "f32", None, pt, np.array([1], np.int32), P)
    assert scales[0, 0, 0] == np.float16(1.0).view(np.uint16)
    # codes 7, -7 -> 0x7 | 0x9 << 4;  3, -1 -> 0x3 | 0xF << 4
    assert codes[0, 0, 0, 0] == 0x97 and codes[0, 0, 0, 1] == 0xF3
    assert not codes[0, 0, 0, 2:].any()


@pytest.mark.parametrize("kv_dtype", ["bf16", "i8"])
def test_index_roundtrip_error_bound(kv_dtype):
    wl = synth.make_custom(B=2, Hq=8, Hkv=2, lens=(70, 33), kv_dtype=kv_dtype, q_dtype="bf16",
                           mode="sals", page_table="random", seed=4)
    codes, scales = oracle.sals_index(wl.k, kv_dtype, wl.k_scale, wl.page_table, wl.seq_lens, wl.proj)
    c = _decode_codes(codes).astype(np.float64)
    s = synth.f16_to_f32(scales).astype(np.float64)
    if kv_dtype == "bf16":
        kf = synth.bf16_to_f32(wl.k).astype(np.float64)
    else:
        kf = wl.k.astype(np.float64) * synth.f16_to_f32(wl.k_scale).astype(np.float64)[..., None]
    kp = kf @ wl.proj.astype(np.float64)  # [P,S,Hkv,r] in double
    for b in range(wl.B):
        for t in range(int(wl.seq_lens[b])):
            pp, sl = wl.page_table[b, t // 16], t % 16
            for h in range(wl.Hkv):
                sc = s[pp, sl, h]
                err = np.abs(kp[pp, sl, h] - c[pp, sl, h] * sc)
                # half-step rounding, widened by the fp32 accumulation and fp16 scale rounding
                assert np.all(err <= 0.5 * sc + 1e-3 * np.abs(kp[pp, sl, h]).max() + 1e-6)
                assert np.abs(c[pp, sl, h]).max() == 7
                assert np.argmax(np.abs(c[pp, sl, h])) == np.argmax(np.abs(kp[pp, sl, h])) or \
                    np.abs(c[pp, sl, h][np.argmax(np.abs(kp[pp, sl, h]))]) == 7


def test_unquantised_identity_projection_is_exact_block_lse():
    """rank = d, P = I and float keys: the block score is logsumexp(tau * qbar . k_t)
    over the block's valid tokens (textbook, via scipy)."""
    wl = synth.make_custom(B=2, Hq=8, Hkv=2, lens=(200, 65), kv_dtype="f32", q_dtype="f32",
                           mode="sals", page_table="random", seed=5)
    I = np.eye(128, dtype=np.float32)
    sc = oracle.sals_scores_float(wl.q, "f32", wl.k, I, wl.page_table, wl.seq_lens, 64,
                                  wl.lse_scale)
    Q = wl.q.astype(np.float64)
    K = wl.k.astype(np.float64)
    for b in range(wl.B):
        L = int(wl.seq_lens[b])
        keys = K[wl.page_table[b, :wl.n_pages(b)]].reshape(-1, 2, 128)[:L]
        for h in range(2):
            qbar = Q[b, 4 * h:4 * h + 4].mean(axis=0)
            z = wl.lse_scale * (keys[:, h] @ qbar)
            for u in range(-(-L // 64)):
                want = scipy.special.logsumexp(z[64 * u:64 * (u + 1)])
                assert abs(sc[b, h, u] - want) <= 1e-12 * max(1.0, abs(want))
            assert np.all(sc[b, h, -(-L // 64):] == -np.inf)


def test_codes_scorer_equals_float_scorer_on_dequantised_keys():
    wl = synth.make_custom(B=1, Hq=4, Hkv=1, lens=(130,), kv_dtype="bf16", q_dtype="bf16",
                           mode="sals", seed=6)
    codes, scales = oracle.sals_index(wl.k, "bf16", None, wl.page_table, wl.seq_lens, wl.proj)
    deq = (_decode_codes(codes).astype(np.float32) * synth.f16_to_f32(scales)[..., None]).astype(np.float32)
    a, ab = oracle.sals_scores(wl.q, "bf16", codes, scales, wl.proj, wl.page_table, wl.seq_lens, 1,
                               64, wl.lse_scale)
    b = oracle.sals_scores_float(wl.q, "bf16", deq, wl.proj, wl.page_table, wl.seq_lens, 64,
                                 wl.lse_scale)
    assert np.array_equal(a, b)
    fin = np.isfinite(a)
    assert np.all(ab[fin] > 0)


def test_block_lse_bounds_and_single_token_block():
    """max_t z_t <= LSE <= max_t z_t + log(n_valid); a 1-token block gives LSE = z."""
    wl = synth.make_custom(B=1, Hq=2, Hkv=1, lens=(64 * 3 + 1,), kv_dtype="f32", q_dtype="f32",
                           mode="sals", seed=7)
    keys = np.ascontiguousarray(wl.k[..., :16])
    proj = np.eye(16, dtype=np.float32)
    proj = np.vstack([proj, np.zeros((112, 16), np.float32)])
    sc = oracle.sals_scores_float(wl.q, "f32", keys, proj, wl.page_table, wl.seq_lens, 64, 0.3)
    qbar = wl.q[0].astype(np.float64).mean(axis=0)[:16]
    kk = keys.reshape(-1, 1, 16)[:193, 0].astype(np.float64)
    z = 0.3 * (kk @ qbar)
    for u in range(3):
        zu = z[64 * u:64 * (u + 1)]
        assert zu.max() - 1e-12 <= sc[0, 0, u] <= zu.max() + np.log(64) + 1e-12
    assert abs(sc[0, 0, 3] - z[192]) <= 1e-12 * max(1, abs(z[192]))
