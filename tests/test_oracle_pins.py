"""Pins for the float64 oracle: checks against things other than itself.

* 16-bit decoding against numpy's float16 and torch's bfloat16 conversions
  over all 65536 bit patterns.
* Closed forms: one key (O = v0, LSE = s0), identical keys (O = mean v,
  LSE = s + ln L), two keys (logistic weights), one dominant key.
* Library routine: torch's scaled_dot_product_attention and
  scipy's logsumexp in float64 on the CPU, dense and paged, GQA 1/2/4/8.
* Invariants: value bounds, LSE bounds, physical page permutation, NaN
  poison outside the valid keys, split count (online recurrence + combine).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle import planner
from split_kv_paged_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def f64(bits, dtype):
    return W.from_bits(bits, dtype).astype(np.float64)


# ---------------------------------------------------------------- decoding --

def test_decode_fp16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode16(bits, "fp16")
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode16(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


# ------------------------------------------------------------ closed forms --

def _dense(q, k, v, dtype="fp16", scale=None):
    return oracle.dense_attention(W.to_bits(q, dtype), W.to_bits(k, dtype), W.to_bits(v, dtype),
                                  dtype, scale=scale)


def test_single_key_gives_value_row():
    # integer-valued q, k so the score is exact: q.k = 1*3 + 2*(-1) = 1
    d = 8
    q = np.zeros((1, 1, d), np.float32); q[0, 0, :2] = [1, 2]
    k = np.zeros((1, 1, d), np.float32); k[0, 0, :2] = [3, -1]
    v = np.random.default_rng(0).standard_normal((1, 1, d)).astype(np.float32)
    for dt in ("fp16", "bf16"):
        out, lse = _dense(q, k, v, dt, scale=0.5)
        assert np.array_equal(out[0, 0], f64(W.to_bits(v, dt), dt)[0, 0])
        assert lse[0, 0] == 0.5


def test_identical_keys_give_mean_value():
    rng = np.random.default_rng(1)
    d, L = 16, 37
    q = rng.standard_normal((2, 3, d)).astype(np.float32)
    k = np.repeat(rng.standard_normal((1, 1, d)).astype(np.float32), L, axis=1)
    v = rng.standard_normal((1, L, d)).astype(np.float32)
    out, lse = _dense(q, k, v, "fp16")
    vb = f64(W.to_bits(v, "fp16"), "fp16")[0]
    qb = f64(W.to_bits(q, "fp16"), "fp16")
    kb = f64(W.to_bits(k, "fp16"), "fp16")[0, 0]
    for h in range(2):
        for i in range(3):
            np.testing.assert_allclose(out[h, i], vb.mean(axis=0), rtol=0, atol=1e-13)
            s = (qb[h, i] @ kb) / math.sqrt(d)
            assert abs(lse[h, i] - (s + math.log(L))) < 1e-12


def test_two_keys_logistic_weights():
    rng = np.random.default_rng(2)
    d = 32
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = rng.standard_normal((1, 2, d)).astype(np.float32)
    v = rng.standard_normal((1, 2, d)).astype(np.float32)
    out, lse = _dense(q, k, v, "bf16", scale=0.3)
    qb, kb, vb = (f64(W.to_bits(x, "bf16"), "bf16") for x in (q, k, v))
    s0 = 0.3 * float(qb[0, 0] @ kb[0, 0])
    s1 = 0.3 * float(qb[0, 0] @ kb[0, 1])
    w0 = 1.0 / (1.0 + math.exp(s1 - s0))
    w1 = 1.0 / (1.0 + math.exp(s0 - s1))
    np.testing.assert_allclose(out[0, 0], w0 * vb[0, 0] + w1 * vb[0, 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse[0, 0], max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))),
                               rtol=0, atol=1e-12)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(3)
    d, L, hot = 64, 50, 17
    q = rng.standard_normal((1, 1, d)).astype(np.float32)
    k = 0.05 * rng.standard_normal((1, L, d)).astype(np.float32)
    k[0, hot] = 8.0 * q[0, 0]
    v = rng.standard_normal((1, L, d)).astype(np.float32)
    out, lse = _dense(q, k, v, "fp16")
    vb = f64(W.to_bits(v, "fp16"), "fp16")
    qb, kb = f64(W.to_bits(q, "fp16"), "fp16"), f64(W.to_bits(k, "fp16"), "fp16")
    s_hot = float(qb[0, 0] @ kb[0, hot]) / 8.0
    np.testing.assert_allclose(out[0, 0], vb[0, hot], atol=1e-6)
    assert s_hot <= lse[0, 0] <= s_hot + 1e-6


def test_empty_sequence_gives_zero_and_minus_inf():
    wl = W.make_paged(5, "bf16", 3, 2, 4, 2, 16, 4, [0, 5, 0], spare_pages=1)
    out, lse = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.cache_seqlens, "bf16")
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.all(np.isneginf(lse[0])) and np.all(np.isneginf(lse[2]))
    assert np.all(np.isfinite(lse[1]))


# ---------------------------------------------------------- library routine --

def _sdpa(qb, kb, vb, scale):
    """torch float64 CPU attention; q [H, n, d], k/v [Hkv, L, d] (GQA by repeat)."""
    G = qb.shape[0] // kb.shape[0]
    q = torch.from_numpy(qb)
    k = torch.from_numpy(kb).repeat_interleave(G, dim=0)
    v = torch.from_numpy(vb).repeat_interleave(G, dim=0)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=scale)
    s = torch.matmul(q, k.transpose(-1, -2)) * scale
    lse = scipy.special.logsumexp(s.numpy(), axis=-1)
    return out.numpy(), lse


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
@pytest.mark.parametrize("hq,hkv,qlen,L,d", [(4, 4, 1, 1, 8), (4, 2, 3, 9, 8), (8, 2, 2, 33, 64),
                                             (16, 2, 1, 70, 128), (8, 1, 4, 5, 24)])
def test_dense_matches_torch_sdpa(dtype, hq, hkv, qlen, L, d):
    wl = W.make_dense(11 + L, dtype, hq, hkv, qlen, L, d)
    out, lse = oracle.dense_attention(wl.q, wl.k, wl.v, dtype)
    ro, rl = _sdpa(f64(wl.q, dtype), f64(wl.k, dtype), f64(wl.v, dtype), 1.0 / math.sqrt(d))
    np.testing.assert_allclose(out, ro, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("dtype,G,d,page", [("bf16", 4, 128, 16), ("fp16", 2, 64, 16),
                                             ("bf16", 8, 64, 8), ("fp16", 1, 32, 5)])
def test_paged_matches_torch_sdpa_on_gathered_kv(dtype, G, d, page):
    hkv, B, qlen = 2, 3, 2
    lens = [1, 2 * page + 3, 3 * page]
    wl = W.make_paged(21 + G, dtype, B, qlen, G * hkv, hkv, d, page, lens, spare_pages=2)
    out, lse = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.cache_seqlens, dtype)
    kc, vc = f64(wl.k_cache, dtype), f64(wl.v_cache, dtype)
    qf = f64(wl.q, dtype)
    for b in range(B):
        L = lens[b]
        pages = wl.block_table[b, :(L + page - 1) // page]
        kseq = kc[pages].reshape(-1, hkv, d)[:L].transpose(1, 0, 2)  # [Hkv, L, d]
        vseq = vc[pages].reshape(-1, hkv, d)[:L].transpose(1, 0, 2)
        ro, rl = _sdpa(qf[b].transpose(1, 0, 2).copy(), kseq.copy(), vseq.copy(),
                       1.0 / math.sqrt(d))
        np.testing.assert_allclose(out[b].transpose(1, 0, 2), ro, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b], rl, rtol=1e-12, atol=1e-12)


# ------------------------------------------------------------------ causal --
# Bottom-right alignment: the q_len queries are the last q_len positions, so
# query i sees keys j <= L - q_len + i.  The mask below is built from that
# sentence alone and handed to torch's attention in float64.

def _causal_mask(qlen, L):
    i = np.arange(qlen)[:, None]
    j = np.arange(L)[None, :]
    return j <= L - qlen + i


def _sdpa_masked(qb, kb, vb, scale, mask):
    """torch float64 attention with a boolean [n, L] mask; rows that see no
    key come back as None."""
    G = qb.shape[0] // kb.shape[0]
    q = torch.from_numpy(qb)
    k = torch.from_numpy(kb).repeat_interleave(G, dim=0)
    v = torch.from_numpy(vb).repeat_interleave(G, dim=0)
    m = torch.from_numpy(mask)
    live = mask.any(axis=1)
    out = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=m, scale=scale)
    s = (torch.matmul(q, k.transpose(-1, -2)) * scale).numpy()
    s = np.where(mask[None], s, -np.inf)
    lse = np.full(s.shape[:2], -np.inf)
    lse[:, live] = scipy.special.logsumexp(s[:, live], axis=-1)
    return out.numpy(), lse, live


@pytest.mark.parametrize("hq,hkv,qlen,L,d", [(4, 2, 3, 9, 8), (8, 2, 4, 33, 64), (8, 8, 8, 8, 16),
                                             (4, 1, 6, 3, 24), (2, 2, 5, 70, 128)])
def test_causal_dense_matches_torch_with_bottom_right_mask(hq, hkv, qlen, L, d):
    wl = W.make_dense(31 + L + qlen, "bf16", hq, hkv, qlen, L, d)
    out, lse = oracle.dense_attention(wl.q, wl.k, wl.v, "bf16", causal=True)
    mask = _causal_mask(qlen, L)
    ro, rl, live = _sdpa_masked(f64(wl.q, "bf16"), f64(wl.k, "bf16"), f64(wl.v, "bf16"),
                                1.0 / math.sqrt(d), mask)
    np.testing.assert_allclose(out[:, live], ro[:, live], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse[:, live], rl[:, live], rtol=1e-12, atol=1e-12)
    assert np.all(out[:, ~live] == 0) and np.all(np.isneginf(lse[:, ~live]))


@pytest.mark.parametrize("G,qlen,page", [(4, 4, 16), (1, 8, 16), (2, 3, 5)])
def test_causal_paged_matches_torch_on_gathered_kv(G, qlen, page):
    hkv, B, d = 2, 3, 32
    lens = [2, qlen, 2 * page + 3]  # first one shorter than q_len: an empty row
    wl = W.make_paged(41 + G + qlen, "fp16", B, qlen, G * hkv, hkv, d, page, lens, spare_pages=2)
    out, lse = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.cache_seqlens, "fp16", causal=True)
    kc, vc = f64(wl.k_cache, "fp16"), f64(wl.v_cache, "fp16")
    qf = f64(wl.q, "fp16")
    for b in range(B):
        L = lens[b]
        pages = wl.block_table[b, :(L + page - 1) // page]
        kseq = kc[pages].reshape(-1, hkv, d)[:L].transpose(1, 0, 2).copy()
        vseq = vc[pages].reshape(-1, hkv, d)[:L].transpose(1, 0, 2).copy()
        ro, rl, live = _sdpa_masked(qf[b].transpose(1, 0, 2).copy(), kseq, vseq,
                                    1.0 / math.sqrt(d), _causal_mask(qlen, L))
        ob = out[b].transpose(1, 0, 2)  # [Hq, qlen, d]
        np.testing.assert_allclose(ob[:, live], ro[:, live], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(lse[b][:, live], rl[:, live], rtol=1e-12, atol=1e-12)
        assert np.all(ob[:, ~live] == 0) and np.all(np.isneginf(lse[b][:, ~live]))


def test_causal_closed_forms():
    """q_len = L: query 0 sees key 0 only (O = v_0 exactly, LSE = s_00);
    query 1 sees keys 0 and 1 (logistic weights); the last query sees all."""
    rng = np.random.default_rng(5)
    L = 4
    q = rng.standard_normal((1, L, 8)).astype(np.float32)
    k = rng.standard_normal((1, L, 8)).astype(np.float32)
    v = rng.standard_normal((1, L, 8)).astype(np.float32)
    qb, kb, vb = (W.to_bits(x, "fp16") for x in (q, k, v))
    out, lse = oracle.dense_attention(qb, kb, vb, "fp16", scale=0.5, causal=True)
    qf, kf, vf = f64(qb, "fp16")[0], f64(kb, "fp16")[0], f64(vb, "fp16")[0]
    s = 0.5 * qf @ kf.T
    assert np.array_equal(out[0, 0], vf[0])
    assert lse[0, 0] == s[0, 0]
    w1 = 1.0 / (1.0 + math.exp(s[1, 1] - s[1, 0]))
    np.testing.assert_allclose(out[0, 1], w1 * vf[0] + (1 - w1) * vf[1], rtol=1e-13, atol=1e-14)
    full, full_lse = oracle.dense_attention(qb, kb, vb, "fp16", scale=0.5)
    assert np.array_equal(out[0, L - 1], full[0, L - 1]) and lse[0, L - 1] == full_lse[0, L - 1]


def test_causal_with_one_query_changes_nothing():
    wl = W.make_paged(51, "bf16", 3, 1, 8, 2, 64, 16, [1, 17, 100], spare_pages=1)
    a = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.cache_seqlens,
                               "bf16")
    b = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table, wl.cache_seqlens,
                               "bf16", causal=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_causal_split_partials_combine_to_direct():
    wl = W.make_paged(61, "bf16", 2, 5, 8, 2, 64, 16, [3, 77], spare_pages=1)
    ref_o, ref_l = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                          wl.cache_seqlens, "bf16", causal=True)
    for S in (1, 2, 3, 6):
        C = oracle.split_keys_for(77, S)
        o, l = oracle.paged_split_partials(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                           wl.cache_seqlens, "bf16", S, C, block=16, causal=True)
        out, lse = oracle.combine(o, l)
        n = 2 * 5 * 8
        np.testing.assert_allclose(out, ref_o.reshape(n, 64), rtol=1e-12, atol=1e-12)
        ref = ref_l.transpose(0, 2, 1).reshape(n)
        live = ~np.isneginf(ref)
        np.testing.assert_allclose(lse[live], ref[live], rtol=1e-12, atol=1e-12)
        assert np.array_equal(np.isneginf(lse), ~live)


# --------------------------------------------------------------- invariants --

def test_value_and_lse_bounds():
    wl = W.make_paged(31, "fp16", 4, 2, 8, 4, 64, 16, [1, 17, 100, 257], outlier_p=0.05)
    out, lse = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.cache_seqlens, "fp16")
    kc, vc = f64(wl.k_cache, "fp16"), f64(wl.v_cache, "fp16")
    qf = f64(wl.q, "fp16")
    for b in range(4):
        L = int(wl.cache_seqlens[b])
        pages = wl.block_table[b, :(L + 15) // 16]
        kseq = kc[pages].reshape(-1, 4, 64)[:L]
        vseq = vc[pages].reshape(-1, 4, 64)[:L]
        for i in range(2):
            for h in range(8):
                vv = vseq[:, h // 2]
                o = out[b, i, h]
                assert np.all(o >= vv.min(axis=0) - 1e-12) and np.all(o <= vv.max(axis=0) + 1e-12)
                s = kseq[:, h // 2] @ qf[b, i, h] / 8.0
                assert s.max() - 1e-12 <= lse[b, h, i] <= s.max() + math.log(L) + 1e-12


def _permute_pool(wl, seed):
    """Same logical cache, different physical page ids."""
    rng = np.random.default_rng(seed)
    n = wl.k_cache.shape[0]
    perm = rng.permutation(n)              # new id of old page p is perm[p]
    kc = np.empty_like(wl.k_cache); vc = np.empty_like(wl.v_cache)
    kc[perm] = wl.k_cache; vc[perm] = wl.v_cache
    return kc, vc, perm[wl.block_table].astype(np.int32)


def test_page_permutation_invariance_is_exact():
    wl = W.make_paged(41, "bf16", 5, 1, 16, 4, 128, 16, [3, 16, 31, 64, 200], spare_pages=3)
    out, lse = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.cache_seqlens, "bf16")
    kc, vc, bt = _permute_pool(wl, 7)
    out2, lse2 = oracle.paged_attention(wl.q, kc, vc, bt, wl.cache_seqlens, "bf16")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_poison_outside_valid_keys_is_never_read():
    wl = W.make_paged(51, "fp16", 3, 1, 4, 2, 64, 16, [5, 16, 33], spare_pages=2)
    out, lse = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.cache_seqlens, "fp16")
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse))
    # replace the poison with ordinary numbers: nothing changes
    kc, vc = wl.k_cache.copy(), wl.v_cache.copy()
    kc[kc == W.NAN16["fp16"]] = W.to_bits(np.float32(3.0), "fp16")
    vc[vc == W.NAN16["fp16"]] = W.to_bits(np.float32(-2.0), "fp16")
    out2, lse2 = oracle.paged_attention(wl.q, kc, vc, wl.block_table, wl.cache_seqlens, "fp16")
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_gqa_head_permutation_within_group_permutes_outputs():
    wl = W.make_paged(61, "bf16", 2, 1, 8, 2, 64, 16, [40, 77])
    out, lse = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.cache_seqlens, "bf16")
    perm = np.array([2, 0, 3, 1, 5, 7, 4, 6])  # stays inside groups {0..3}, {4..7}
    q2 = wl.q[:, :, perm]
    out2, lse2 = oracle.paged_attention(q2, wl.k_cache, wl.v_cache, wl.block_table,
                                        wl.cache_seqlens, "bf16")
    assert np.array_equal(out2, out[:, :, perm]) and np.array_equal(lse2, lse[:, perm])


@pytest.mark.parametrize("block", [1, 5, 16, 64])
def test_split_partials_and_combine_equal_direct(block):
    wl = W.make_paged(71, "fp16", 4, 2, 8, 2, 64, 16, [1, 15, 129, 300], outlier_p=0.02)
    out, lse = oracle.paged_attention(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                      wl.cache_seqlens, "fp16")
    n = 4 * 2 * 8
    ref_o = out.reshape(n, 64)
    ref_l = lse.transpose(0, 2, 1).reshape(n)
    cases = [(S, oracle.split_keys_for(300, S)) for S in list(range(1, 17)) + [40]]
    cases += [(43, 7), (3, 100), (1, 300), (2, 1000)]  # other split lengths covering L
    for S, C in cases:
        o, l = oracle.paged_split_partials(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                           wl.cache_seqlens, "fp16", S, C, block=block)
        co, cl = oracle.combine(o, l)
        np.testing.assert_allclose(co, ref_o, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(cl, ref_l, rtol=1e-12, atol=1e-12)


def test_split_length_rule():
    assert oracle.split_keys_for(16384, 14) == 16 * 74    # ceil(1024/14) = 74 units
    assert oracle.split_keys_for(1100, 1) == 1104         # 69 units of 16
    assert oracle.split_keys_for(1, 4) == 16              # at least one granule
    assert oracle.split_keys_for(0, 3) == 16
    with pytest.raises(ValueError):                        # splits must cover every key
        wl = W.make_paged(72, "fp16", 1, 1, 2, 1, 16, 16, [40])
        oracle.paged_split_partials(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                    wl.cache_seqlens, "fp16", 2, 16)


def test_split_ranges_cover_keys_once_and_empty_splits_are_neutral():
    # L = 1 with 4 splits of 16: split 0 holds the key, the other three are empty
    wl = W.make_paged(81, "bf16", 1, 1, 2, 1, 16, 16, [1])
    o, l = oracle.paged_split_partials(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                       wl.cache_seqlens, "bf16", 4, 16)
    assert np.all(np.isfinite(l[0])) and np.all(np.isneginf(l[1:]))
    assert np.all(o[1:] == 0)
    np.testing.assert_array_equal(o[0, 0], f64(wl.v_cache, "bf16")[wl.block_table[0, 0], 0, 0])
    # a short sequence only fills the first splits of a long batch's split length
    wl = W.make_paged(82, "bf16", 2, 1, 2, 1, 16, 16, [20, 100])
    o, l = oracle.paged_split_partials(wl.q, wl.k_cache, wl.v_cache, wl.block_table,
                                       wl.cache_seqlens, "bf16", 4, 32)
    # rows of sequence 0 are n = 0, 1; keys 0..19 -> split 0 has 20 keys, split 1..3 empty
    assert np.all(np.isfinite(l[0, :2])) and np.all(np.isneginf(l[1:, :2]))
    assert np.all(np.isfinite(l[:, 2:]))  # 100 keys reach split 3 (96..99)


def test_dense_split_matches_dense_direct():
    wl = W.make_dense(91, "fp16", 4, 2, 3, 1025, 24)
    out, lse = oracle.dense_attention(wl.q, wl.k, wl.v, "fp16")
    for S in (1, 3, 7):
        o, l = oracle.dense_split_partials(wl.q, wl.k, wl.v, "fp16", S,
                                           oracle.split_keys_for(1025, S), block=32)
        co, cl = oracle.combine(o, l)
        np.testing.assert_allclose(co, out.reshape(12, 24), rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(cl, lse.reshape(12), rtol=1e-12, atol=1e-12)


def test_combine_closed_forms():
    d = 4
    a = np.array([1.0, 2.0, 3.0, 4.0]); b = np.array([-1.0, 0.5, 0.0, 8.0])
    # equal weights: average, LSE + ln 2
    o, l = oracle.combine(np.stack([a, b])[:, None, :], np.array([[0.7], [0.7]]))
    np.testing.assert_allclose(o[0], (a + b) / 2, atol=1e-15)
    assert abs(l[0] - (0.7 + math.log(2))) < 1e-15
    # an empty partial has no weight
    o, l = oracle.combine(np.stack([a, np.zeros(d)])[:, None, :], np.array([[1.5], [-np.inf]]))
    np.testing.assert_array_equal(o[0], a)
    assert l[0] == 1.5
    # all empty: zero output, -inf
    o, l = oracle.combine(np.zeros((3, 1, d)), np.full((3, 1), -np.inf))
    assert np.all(o == 0) and np.isneginf(l[0])
    # weights e^1 : e^0
    o, l = oracle.combine(np.stack([a, b])[:, None, :], np.array([[1.0], [0.0]]))
    w = 1.0 / (1.0 + math.exp(-1.0))
    np.testing.assert_allclose(o[0], w * a + (1 - w) * b, atol=1e-15)


# ------------------------------------------------------------ planner rules --

def _golden():
    with open(os.path.join(GOLDEN, "planner_examples.json")) as f:
        return json.load(f)


@pytest.mark.parametrize("case", _golden()["should_pack_gqa"], ids=lambda c: c["note"][:40])
def test_planner_pack_rule_pinned(case):
    assert planner.should_pack_gqa(case["varlen_q"], case["seqlen_q"], case["qhead_per_khead"],
                                   case["block_m"]) == case["expect"]


@pytest.mark.parametrize("case", _golden()["num_splits_heuristic"], ids=lambda c: c["note"][:40])
def test_planner_split_rule_pinned(case):
    assert planner.num_splits_heuristic(case["total_mblocks"], case["num_sms"],
                                        case["num_n_blocks"]) == case["expect"]


@pytest.mark.parametrize("case", _golden()["plan"], ids=lambda c: c["note"][:40])
def test_planner_plan_pinned(case):
    got = planner.plan(case["batch"], case["seqlen_q"], case["num_heads_q"],
                       case["num_heads_kv"], case["max_seqlen_k"], case["num_sms"],
                       case["block_m"], case["block_n"], case["num_splits"], case["pack_gqa"])
    assert got == (case["expect_splits"], case["expect_pack"])


@pytest.mark.parametrize("batch,hkv,max_L", [(1, 4, 4096), (4, 4, 16384), (3, 8, 2048),
                                              (32, 8, 1024), (2, 1, 8192)])
def test_planner_unit_tile_counts_thread_blocks(batch, hkv, max_L):
    """With a thread block carrying 64 packed rows, 64 rows a head count as
    one unit, exactly as 16 rows do with 16-row blocks; with 16-row blocks
    the same 64 rows count as four units, as four heads of 16 rows would."""
    base = planner.plan(batch, 1, 16 * hkv, hkv, max_L, 256, 16, 128)          # 16 rows, 1 unit
    wide = planner.plan(batch, 8, 8 * hkv, hkv, max_L, 256, 16, 128, unit_block_m=64)
    assert wide == base
    four = planner.plan(batch, 1, 16 * 4 * hkv, 4 * hkv, max_L, 256, 16, 128)  # 4 units
    assert planner.plan(batch, 8, 8 * hkv, hkv, max_L, 256, 16, 128) == four


def test_planner_wave_efficiency_brute_force():
    """The chosen split count is the smallest s whose last-wave fill is within
    85% of the best, found here by exhaustive rational arithmetic."""
    from fractions import Fraction
    for units in (1, 3, 7, 16, 50, 100, 190):
        for sms in (132, 256):
            for nblocks in (5, 9, 64, 128, 300):
                if units >= 0.8 * sms:
                    continue
                eff = []
                for s in range(1, min(128, nblocks) + 1):
                    w = Fraction(units * s, sms)
                    eff.append(w / math.ceil(w))
                best = max(eff)
                want = next(s for s in range(1, len(eff) + 1)
                            if eff[s - 1] >= Fraction(85, 100) * best)
                assert planner.num_splits_heuristic(units, sms, nblocks) == want
