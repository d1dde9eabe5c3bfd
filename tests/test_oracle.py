"""Pins for the CPU oracle (no GPU).

Each test ties the oracle to something other than itself: the figures the
pages print, closed forms, special cases that reduce to a library routine
(PyTorch's fp64 scaled_dot_product_attention on the CPU), invariants the
pages state (MHA and MQA as the two ends of GQA; GQA equals MHA with every
K/V head repeated G times), and brute force on tiny shapes.  A last group
plants plausible mistakes in a copy of the reference and checks that the pins
catch every one of them.
"""
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import np_oracle

HERE = os.path.dirname(os.path.abspath(__file__))


def rand(rng, *shape):
    return rng.standard_normal(shape)


def sdpa_ref(q, k, v, q_start, kv_len, causal, scale, window=0):
    """PyTorch fp64 SDPA (CPU, math path) row by row with an explicit mask.

    q [B,Sq,H,d], k/v [B,K,Sk,d]; enable_gqa broadcasts KV head h // G.
    window > 0 adds the band j > qpos - window to the mask."""
    B, Sq, H, d = q.shape
    K, Sk = k.shape[1], k.shape[2]
    out = np.full(q.shape, np.nan)
    for b in range(B):
        qt = torch.from_numpy(q[b]).permute(1, 0, 2).unsqueeze(0)        # [1,H,Sq,d]
        kt = torch.from_numpy(k[b]).unsqueeze(0)                          # [1,K,Sk,d]
        vt = torch.from_numpy(v[b]).unsqueeze(0)
        pos = q_start[b] + np.arange(Sq)[:, None]
        j = np.arange(Sk)[None, :]
        allowed = j < min(kv_len[b], Sk)
        if causal:
            allowed = allowed & (j <= pos)
        if window > 0:
            allowed = allowed & (j > pos - window)
        mask = torch.from_numpy(np.broadcast_to(allowed, (Sq, Sk)).copy())
        o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale,
                                           enable_gqa=(H != K))
        o = o[0].permute(1, 0, 2).numpy()
        rows_ok = np.broadcast_to(allowed, (Sq, Sk)).any(axis=1)
        out[b][rows_ok] = o[rows_ok]
    return out


# ---------------------------------------------------------------------------
# cache size: the figures printed on the pages
# ---------------------------------------------------------------------------

def _golden_cases():
    cases = []
    with open(os.path.join(HERE, "golden", "kv_cache_size.txt")) as f:
        for line in f:
            line = line.strip()
            if not line.startswith("case "):
                continue
            parts = line.split()
            kv = dict(p.split("=", 1) for p in parts[2:])
            cases.append((parts[1], kv))
    return cases


@pytest.mark.parametrize("name,kv", _golden_cases(), ids=[c[0] for c in _golden_cases()])
def test_cache_size_matches_printed_figures(oracle_lib, name, kv):
    elems = oracle.kv_cache_elems(int(kv["layers"]), int(kv["kv_heads"]), int(kv["head_dim"]),
                                  int(kv["seq_len"]), int(kv["batch"]))
    value = elems * int(kv["bytes_per_elem"]) / float(kv["unit"])
    printed = float(kv["printed"])
    assert abs(value - printed) < 10.0 ** (-int(kv["digits"])), (name, value, printed)


def test_cache_size_exact_counts(oracle_lib):
    # concept page 关键参数 #2: 2*64*2048*128*80 and 2*8*2048*128*80
    assert oracle.kv_cache_elems(80, 64, 128, 2048, 1) == 2_684_354_560
    assert oracle.kv_cache_elems(80, 8, 128, 2048, 1) == 335_544_320
    # the MHA/GQA ratio is H/K
    assert oracle.kv_cache_elems(80, 64, 128, 2048, 1) // oracle.kv_cache_elems(80, 8, 128, 2048, 1) == 8


@pytest.mark.parametrize("K,d,expect", [(8, 128, 2048), (64, 128, 16384), (1, 128, 256), (2, 64, 256)])
def test_cache_elems_per_token(oracle_lib, K, d, expect):
    assert oracle.cache_elems_per_token(K, d) == expect
    assert oracle.kv_cache_elems(1, K, d, 1, 1) == expect


# ---------------------------------------------------------------------------
# attention: library routine, brute force, special cases
# ---------------------------------------------------------------------------

SHAPES = [
    # B, Sq, H, K, d, Sk
    (1, 1, 1, 1, 4, 1),
    (2, 3, 4, 2, 8, 9),
    (1, 5, 8, 1, 16, 12),   # MQA
    (2, 4, 6, 6, 8, 7),     # MHA
    (3, 2, 8, 4, 64, 33),
    (1, 8, 8, 2, 64, 8),
]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("causal", [False, True])
def test_c_oracle_vs_torch_sdpa_and_numpy(oracle_lib, shape, causal):
    B, Sq, H, K, d, Sk = shape
    rng = np.random.default_rng(hash(shape) % 2**32 + causal)
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    kv_len = rng.integers(1, Sk + 1, size=B).astype(np.int32)
    # causal rows: the last query sits on the last valid key
    q_start = np.maximum(kv_len - Sq, 0).astype(np.int32) if causal else np.zeros(B, np.int32)
    scale = 1.0 / math.sqrt(d)
    got = oracle.attention(q, k, v, q_start, kv_len, causal, scale)
    ref_t = sdpa_ref(q, k, v, q_start, kv_len, causal, scale)
    ref_n = np_oracle.gqa_reference(q, k, v, q_start, kv_len, causal, scale)
    ok = ~np.isnan(ref_t)
    assert np.array_equal(ok, ~np.isnan(got))
    np.testing.assert_allclose(got[ok], ref_t[ok], rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[ok], ref_n[ok], rtol=0, atol=1e-12)


def test_rows_entry_matches_full(oracle_lib):
    rng = np.random.default_rng(7)
    B, Sq, H, K, d, Sk = 2, 6, 8, 2, 16, 10
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    qs, kl = np.array([2, 4], np.int32), np.array([8, 10], np.int32)
    full = oracle.attention(q, k, v, qs, kl, True, 0.3)
    rows = np.array([[b, i, h] for b in range(B) for i in range(Sq) for h in range(H)], np.int32)
    sel = oracle.attention_rows(q, k, v, qs, kl, True, 0.3, rows)
    assert np.array_equal(sel, full.reshape(-1, d))


def test_mha_end_is_per_head_attention(oracle_lib):
    """K = H (G = 1): each head uses its own K/V head (plain multi-head attention)."""
    rng = np.random.default_rng(11)
    B, H, d, Sk = 2, 4, 8, 6
    q, k, v = rand(rng, B, 1, H, d), rand(rng, B, H, Sk, d), rand(rng, B, H, Sk, d)
    got = oracle.attention(q, k, v, [Sk - 1] * B, [Sk] * B, False, 0.5)
    for b in range(B):
        for h in range(H):
            s = 0.5 * (k[b, h] @ q[b, 0, h])
            w = np.exp(s - s.max())
            np.testing.assert_allclose(got[b, 0, h], (w @ v[b, h]) / w.sum(), atol=1e-13)


def test_mqa_end_shares_one_head(oracle_lib):
    """K = 1: every query head reads the single K/V head."""
    rng = np.random.default_rng(12)
    B, H, d, Sk = 1, 8, 8, 9
    q, k, v = rand(rng, B, 1, H, d), rand(rng, B, 1, Sk, d), rand(rng, B, 1, Sk, d)
    got = oracle.attention(q, k, v, [Sk - 1], [Sk], False, 0.4)
    for h in range(H):
        one = oracle.attention(q[:, :, h:h + 1], k, v, [Sk - 1], [Sk], False, 0.4)
        assert np.array_equal(got[0, 0, h], one[0, 0, 0])


@pytest.mark.parametrize("H,K", [(8, 2), (8, 4), (6, 3), (64, 8), (4, 1)])
def test_gqa_equals_mha_with_repeated_kv(oracle_lib, H, K):
    """Head h reads KV head h // G: GQA equals MHA on K/V repeated G times per head."""
    rng = np.random.default_rng(H * 100 + K)
    B, Sq, d, Sk = 2, 3, 8, 7
    G = H // K
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    qs, kl = np.array([4, 2], np.int32), np.array([7, 5], np.int32)
    gqa = oracle.attention(q, k, v, qs, kl, True, 0.35)
    mha = oracle.attention(q, np.repeat(k, G, axis=1), np.repeat(v, G, axis=1), qs, kl, True, 0.35)
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-13)
    if K > 1 and G > 1:
        # the strided map h % K is a different answer: the pin discriminates
        wrong = oracle.attention(q, np.tile(k, (1, G, 1, 1)), np.tile(v, (1, G, 1, 1)), qs, kl, True, 0.35)
        assert np.max(np.abs(wrong - gqa)) > 1e-3


def test_group_id_recovered_from_constant_v(oracle_lib):
    """V of KV head g is the constant g: every output of head h is h // G."""
    rng = np.random.default_rng(3)
    B, H, K, d, Sk = 2, 16, 4, 8, 11
    q, k = rand(rng, B, 2, H, d), rand(rng, B, K, Sk, d)
    v = np.broadcast_to(np.arange(K, dtype=np.float64)[None, :, None, None], (B, K, Sk, d)).copy()
    out = oracle.attention(q, k, v, [5, 9], [Sk, Sk], True, 0.3)
    for h in range(H):
        np.testing.assert_allclose(out[:, :, h], h // (H // K), rtol=1e-14, atol=1e-14)


def test_single_visible_key_returns_v0_exactly(oracle_lib):
    rng = np.random.default_rng(4)
    B, Sq, H, K, d, Sk = 1, 4, 4, 2, 8, 4
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    out = oracle.attention(q, k, v, [0], [Sk], True, 0.125)
    for h in range(H):
        assert np.array_equal(out[0, 0, h], v[0, h // 2, 0])   # p = e^0 = 1, l = 1
    dec = oracle.attention(q[:, :1], k, v, [0], [1], False, 0.125)
    assert np.array_equal(dec[0, 0, 3], v[0, 1, 0])


def test_zero_query_gives_mean_of_visible_values(oracle_lib):
    rng = np.random.default_rng(5)
    B, H, K, d, Sk = 1, 4, 2, 8, 10
    q = np.zeros((B, 3, H, d))
    k, v = rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    out = oracle.attention(q, k, v, [2], [Sk], True, 0.7)
    for i in range(3):
        for h in range(H):
            np.testing.assert_allclose(out[0, i, h], v[0, h // 2, :2 + i + 1].mean(axis=0), atol=1e-14)


@pytest.mark.parametrize("d", [4, 64, 128])
def test_two_key_closed_form(oracle_lib, d):
    """Two keys: out = v1 * sigmoid(scale (s1 - s2)) + v2 * (1 - sigmoid(...)), scale = 1/sqrt(d)."""
    q = np.zeros((1, 1, 1, d)); q[0, 0, 0, 0] = 1.0
    k = np.zeros((1, 1, 2, d)); k[0, 0, 0, 0] = 3.0; k[0, 0, 1, 0] = -1.0
    v = np.zeros((1, 1, 2, d)); v[0, 0, 0, :] = 1.0; v[0, 0, 1, :] = -2.0
    scale = 1.0 / math.sqrt(d)
    w1 = 1.0 / (1.0 + math.exp(-scale * 4.0))
    out = oracle.attention(q, k, v, [1], [2], False, scale)
    np.testing.assert_allclose(out[0, 0, 0], w1 * 1.0 + (1 - w1) * -2.0, atol=1e-15)


def test_causal_row_equals_decode_over_prefix(oracle_lib):
    """Causal row i (position p + i) sees exactly keys 0..p+i: a decode with ctx = p+i+1."""
    rng = np.random.default_rng(6)
    B, Sq, H, K, d, Sk = 1, 5, 4, 2, 8, 9
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    p = 3
    pre = oracle.attention(q, k, v, [p], [Sk], True, 0.3)
    for i in range(Sq):
        dec = oracle.attention(q[:, i:i + 1], k, v, [p + i], [p + i + 1], False, 0.3)
        assert np.array_equal(pre[0, i], dec[0, 0])


# ---------------------------------------------------------------------------
# sliding window (inference-optimisation page §6.4.1): a row sees only its
# `window` most recent positions
# ---------------------------------------------------------------------------

def _rows_all(B, Sq, H):
    return np.array([[b, i, h] for b in range(B) for i in range(Sq) for h in range(H)], np.int32)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("window", [1, 3, 7, 40])
def test_window_matches_sdpa_band_mask(oracle_lib, causal, window):
    """Against PyTorch's fp64 SDPA with the band j > qpos - window in its mask."""
    rng = np.random.default_rng(31)
    B, Sq, H, K, d, Sk = 2, 6, 4, 2, 8, 21
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    qs, kl = [5, 12], [Sk, 17]
    want = sdpa_ref(q, k, v, qs, kl, causal, 0.31, window)
    got = oracle.attention_rows(q, k, v, qs, kl, causal, 0.31, _rows_all(B, Sq, H), window)
    np.testing.assert_allclose(got, want.reshape(-1, d), rtol=0, atol=1e-12)


def test_window_one_returns_own_value(oracle_lib):
    """window = 1 leaves one key, the row's own position: out = v[qpos] exactly."""
    rng = np.random.default_rng(32)
    B, Sq, H, K, d, Sk = 1, 4, 4, 2, 8, 10
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    got = oracle.attention_rows(q, k, v, [3], [Sk], True, 0.5, _rows_all(B, Sq, H), 1).reshape(Sq, H, d)
    for i in range(Sq):
        for h in range(H):
            assert np.array_equal(got[i, h], v[0, h // 2, 3 + i])


def test_window_covering_every_key_is_no_window(oracle_lib):
    rng = np.random.default_rng(33)
    B, Sq, H, K, d, Sk = 2, 3, 4, 1, 8, 12
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    rows = _rows_all(B, Sq, H)
    full = oracle.attention_rows(q, k, v, [4, 9], [Sk, Sk], True, 0.4, rows)
    wide = oracle.attention_rows(q, k, v, [4, 9], [Sk, Sk], True, 0.4, rows, Sk)
    assert np.array_equal(full, wide)


def test_window_equals_attention_over_the_key_slice(oracle_lib):
    """A decode row with window W equals a plain decode over keys ctx-W .. ctx-1."""
    rng = np.random.default_rng(34)
    H, K, d, ctx, W = 4, 2, 8, 30, 11
    q, k, v = rand(rng, 1, 1, H, d), rand(rng, 1, K, ctx, d), rand(rng, 1, K, ctx, d)
    rows = _rows_all(1, 1, H)
    got = oracle.attention_rows(q, k, v, [ctx - 1], [ctx], False, 0.3, rows, W)
    lo = ctx - W
    want = oracle.attention_rows(q, k[:, :, lo:].copy(), v[:, :, lo:].copy(), [W - 1], [W], False, 0.3, rows)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("window", [2, 9])
def test_window_numpy_oracle_agrees(oracle_lib, window):
    rng = np.random.default_rng(35)
    B, Sq, H, K, d, Sk = 2, 5, 6, 3, 8, 16
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    c = oracle.attention_rows(q, k, v, [2, 7], [Sk, 12], True, 0.35, _rows_all(B, Sq, H), window)
    n = np_oracle.gqa_reference(q, k, v, [2, 7], [Sk, 12], True, 0.35, window)
    np.testing.assert_allclose(c, n.reshape(-1, d), rtol=0, atol=1e-12)


def test_no_visible_key_is_reported(oracle_lib):
    q, k, v = np.ones((1, 1, 2, 4)), np.ones((1, 1, 3, 4)), np.ones((1, 1, 3, 4))
    out = oracle.attention(q, k, v, [0], [0], False, 1.0)
    assert np.isnan(out).all()


# ---------------------------------------------------------------------------
# the rewrites the GPU path relies on are exact (inference-optimisation page
# §9.2.1 online softmax; §10.2 split and merge)
# ---------------------------------------------------------------------------

def test_online_softmax_equals_three_pass(oracle_lib):
    rng = np.random.default_rng(8)
    B, Sq, H, K, d, Sk = 2, 3, 4, 2, 8, 20
    q, k, v = 3 * rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    qs, kl = np.array([10, 17], np.int32), np.array([20, 19], np.int32)
    ref = oracle.attention(q, k, v, qs, kl, True, 0.4)
    onl = np_oracle.online_softmax_attention(q, k, v, qs, kl, True, 0.4)
    np.testing.assert_allclose(onl, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("segment", [1, 3, 16, 64, 1000])
def test_split_merge_equals_three_pass(oracle_lib, segment):
    rng = np.random.default_rng(9)
    B, H, K, d, Sk = 3, 8, 2, 16, 70
    q, k, v = 4 * rand(rng, B, 1, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    kl = np.array([70, 1, 33], np.int32)
    ref = oracle.attention(q, k, v, kl - 1, kl, False, 0.25)
    got = np_oracle.split_merge_attention(q, k, v, kl, 0.25, segment)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------
# cache append and paged gather: pure data movement
# ---------------------------------------------------------------------------

def _coded_rows(B, s, K, d, base=0):
    """Unique float32 codes: row (b, t, g) column c holds b*1e6 + t*1e3 + g*10 + c/1e3."""
    b, t, g, c = np.meshgrid(np.arange(B), np.arange(s), np.arange(K), np.arange(d), indexing="ij")
    return (base + b * 1e6 + t * 1e3 + g * 10 + c / 1e3).astype(np.float32)


def test_append_contiguous_places_every_row(oracle_lib):
    B, s, K, d, S = 3, 5, 2, 4, 12
    cache = np.full((B, K, S, d), -7.0, np.float32)
    new = _coded_rows(B, s, K, d)
    start = np.array([0, 4, 9], np.int32)          # the last one runs past S_max by 2 rows
    dropped = oracle.kv_append(cache, new, start)
    assert dropped == 2 * K
    for b in range(B):
        for g in range(K):
            for p in range(S):
                t = p - start[b]
                if 0 <= t < s:
                    assert np.array_equal(cache[b, g, p], new[b, t, g])
                else:
                    assert (cache[b, g, p] == -7.0).all()


def test_append_paged_and_gather_roundtrip(oracle_lib):
    rng = np.random.default_rng(10)
    B, K, d, bs = 3, 2, 4, 16
    ctx = np.array([1, 16, 37], np.int32)
    nb = (ctx + bs - 1) // bs
    n_pool = int(nb.sum()) + 2
    perm = rng.permutation(n_pool).astype(np.int32)
    table = np.full((B, int(nb.max())), -1, np.int32)
    off = 0
    for b in range(B):
        table[b, :nb[b]] = perm[off:off + nb[b]]
        off += nb[b]
    pool = np.full((n_pool, K, bs, d), -7.0, np.float32)
    s = int(ctx.max())
    new = _coded_rows(B, s, K, d)
    # append each sequence's first ctx[b] tokens one at a time (decode-style)
    for t in range(s):
        for b in range(B):
            if t < ctx[b]:
                oracle.kv_append_paged(pool, new[b:b + 1, t:t + 1], [t], table[b:b + 1])
    got = oracle.gather_paged(pool.astype(np.float64), table, ctx, s)
    for b in range(B):
        for g in range(K):
            assert np.array_equal(got[b, g, :ctx[b]], new[b, :ctx[b], g].astype(np.float64))
            assert np.isnan(got[b, g, ctx[b]:]).all()
    # slots outside every sequence keep the sentinel
    assert (pool == -7.0).sum() == (n_pool * bs - int(ctx.sum())) * K * d


def test_paged_attention_equals_contiguous(oracle_lib):
    rng = np.random.default_rng(13)
    B, H, K, d, bs = 2, 4, 2, 8, 16
    ctx = np.array([5, 40], np.int32)
    nb = (ctx + bs - 1) // bs
    n_pool = int(nb.sum())
    perm = rng.permutation(n_pool).astype(np.int32)
    table = np.full((B, int(nb.max())), -1, np.int32)
    table[0, :nb[0]] = perm[:nb[0]]
    table[1, :nb[1]] = perm[nb[0]:]
    pool_k, pool_v = rand(rng, n_pool, K, bs, d), rand(rng, n_pool, K, bs, d)
    q = rand(rng, B, 1, H, d)
    rows, out = oracle.paged_attention_rows(q, pool_k, pool_v, table, ctx, 0.3)
    S = int(ctx.max())
    kc = oracle.gather_paged(pool_k, table, ctx, S)
    vc = oracle.gather_paged(pool_v, table, ctx, S)
    ref = sdpa_ref(q, np.nan_to_num(kc), np.nan_to_num(vc), ctx - 1, ctx, False, 0.3)
    np.testing.assert_allclose(out.reshape(B, H, d), ref[:, 0], atol=1e-12)


# ---------------------------------------------------------------------------
# paged cache: the oracle's append and gathers against plain NumPy indexing
# (inference-optimisation page §8.2: token t of a sequence lives in physical
# block table[b, t // bs], slot t % bs; the pool is [blocks, K, bs, d])
# ---------------------------------------------------------------------------

def _coded_pool(N, K, bs, d, dtype):
    """A pool whose every element names its (block, head, slot, column): any
    wrong block, head, slot or stride shows as a different value."""
    n, g, s, c = np.meshgrid(np.arange(N), np.arange(K), np.arange(bs), np.arange(d), indexing="ij")
    code = ((n * K + g) * bs + s) * d + c
    if dtype == np.uint16:               # bf16 bit patterns, stored as raw 16-bit words
        return (code % 65000 + 1).astype(np.uint16)
    return (code + 1).astype(dtype)


def _paged_case(rng, bs, K=3, d=5):
    ctx = np.array([1, bs, 3 * bs + 1, 2 * bs - 1], np.int32)
    need = (ctx + bs - 1) // bs
    n_pool = int(need.sum()) + 3                   # three blocks no sequence owns
    perm = rng.permutation(n_pool).astype(np.int32)
    table = np.full((len(ctx), int(need.max()) + 1), -1, np.int32)   # one spare column
    off = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[off:off + nb]
        off += int(nb)
    return ctx, table, n_pool, K, d


def _numpy_gather(pool, table, ctx, S_out, fill):
    """out[b, g, t] = pool[table[b, t // bs], g, t % bs] for t < ctx[b], written
    independently of the oracle with fancy indexing."""
    N, K, bs, d = pool.shape
    out = np.full((len(ctx), K, S_out, d), fill, dtype=pool.dtype)
    for b in range(len(ctx)):
        t = np.arange(min(int(ctx[b]), S_out))
        blk = table[b, t // bs]
        out[b, :, t] = pool[blk, :, t % bs]       # advanced indices first: [t, K, d]
    return out


def _gather_raw_pin_holds(gather):
    """True when `gather(pool, table, ctx, S_out, fill)` equals the NumPy
    indexing on every block size, element type and sequence."""
    rng = np.random.default_rng(31)
    for bs in (1, 4, 16):
        for dtype in (np.uint16, np.float32, np.float64):
            ctx, table, N, K, d = _paged_case(rng, bs)
            pool = _coded_pool(N, K, bs, d, dtype)
            S_out = int(ctx.max()) + 2
            fill = dtype(0) if dtype == np.uint16 else dtype(-1)
            got = gather(pool, table, ctx, S_out, fill)
            if got.shape != (len(ctx), K, S_out, d) or not np.array_equal(got, _numpy_gather(pool, table, ctx, S_out,
                                                                                               fill)):
                return False
    return True


def test_gather_paged_raw_matches_numpy_indexing(oracle_lib):
    assert _gather_raw_pin_holds(oracle.gather_paged_raw)


def test_gather_paged_f64_matches_numpy_indexing(oracle_lib):
    rng = np.random.default_rng(32)
    for bs in (1, 4, 16):
        ctx, table, N, K, d = _paged_case(rng, bs)
        pool = _coded_pool(N, K, bs, d, np.float64)
        S_out = int(ctx.max()) + 2
        got = oracle.gather_paged(pool, table, ctx, S_out)
        want = _numpy_gather(pool, table, ctx, S_out, np.nan)
        assert np.array_equal(got, want, equal_nan=True)


def test_gather_paged_raw_leaves_fill_for_invalid_blocks(oracle_lib):
    """Visible positions whose block id is outside the pool are counted and keep the fill."""
    rng = np.random.default_rng(33)
    ctx, table, N, K, d = _paged_case(rng, 4)
    pool = _coded_pool(N, K, 4, d, np.float32)
    table = table.copy()
    table[2, 1] = N            # one past the pool
    table[3, 0] = -5
    S_out = int(ctx.max())
    out = np.full((len(ctx), K, S_out, d), -1.0, np.float32)
    lib = oracle._load()
    cl = np.ascontiguousarray(ctx, np.int32)
    bad = lib.oracle_gather_paged_raw(pool.ctypes.data, 4, table.ctypes.data, table.shape[1], N, 4,
                                      cl.ctypes.data, len(ctx), K, d, S_out, out.ctypes.data)
    assert bad == 2 * 4 * K    # two 4-token blocks of K heads each
    want = _numpy_gather(pool, np.where((table >= 0) & (table < N), table, 0), ctx, S_out, -1.0)
    want[2, :, 4:8] = -1.0
    want[3, :, 0:4] = -1.0
    assert np.array_equal(out, want)
    with pytest.raises(ValueError):
        oracle.gather_paged_raw(pool, table, ctx, S_out, np.float32(-1))


@pytest.mark.parametrize("bs", [1, 4, 16])
@pytest.mark.parametrize("dtype", [np.uint16, np.float32])
def test_append_paged_matches_numpy_indexing(oracle_lib, bs, dtype):
    """pool[table[b, p // bs], g, p % bs] = new[b, t, g] with p = start[b] + t; every
    other slot keeps its value, and positions past the table are dropped."""
    rng = np.random.default_rng(34 + bs)
    ctx, table, N, K, d = _paged_case(rng, bs)
    B, s_new = len(ctx), 3
    start = np.array([0, bs - 1, 3 * bs - 1, 2 * bs - 3], np.int32)
    pool = _coded_pool(N, K, bs, d, dtype)
    new = (np.arange(B * s_new * K * d).reshape(B, s_new, K, d) % 50000 + 60000).astype(dtype)
    want = pool.copy()
    dropped_want = 0
    for b in range(B):
        for t in range(s_new):
            p = int(start[b]) + t
            blk = table[b, p // bs] if p // bs < table.shape[1] else -1
            if not 0 <= blk < N:
                dropped_want += K
                continue
            want[blk, :, p % bs] = new[b, t]
    got = pool.copy()
    dropped = oracle.kv_append_paged(got, new, start, table)
    assert dropped == dropped_want
    assert np.array_equal(got, want)


# planted mistakes in the paged indexing: each must fail the pins above,
# while an append/gather round trip with the same mistake on both sides
# would still pass

def _mutant_gather(kind):
    def gather(pool, table, ctx, S_out, fill):
        N, K, bs, d = pool.shape
        flat = pool.reshape(-1)
        out = np.full((len(ctx), K, S_out, d), fill, dtype=pool.dtype)
        for b in range(len(ctx)):
            for g in range(K):
                for t in range(min(int(ctx[b]), S_out)):
                    col = t // bs + (1 if kind == "block_column_off_by_one" else 0)
                    blk = int(table[b, col])
                    if not 0 <= blk < N:
                        continue
                    if kind == "head_slot_swapped":          # reads the pool as [N, bs, K, d]
                        row = (blk * bs + t % bs) * K + g
                    else:
                        row = (blk * K + g) * bs + t % bs
                    out[b, g, t] = flat[row * d:(row + 1) * d]
        return out
    return gather


def _byte_stride_gather(pool, table, ctx, S_out, fill):
    """The oracle's raw gather called with a 1-byte element size."""
    pool = np.ascontiguousarray(pool)
    N, K, bs, d = pool.shape
    out = np.full((len(ctx), K, S_out, d), fill, dtype=pool.dtype)
    cl = np.ascontiguousarray(ctx, np.int32)
    bt = np.ascontiguousarray(table, np.int32)
    oracle._load().oracle_gather_paged_raw(pool.ctypes.data, 1, bt.ctypes.data, bt.shape[1], N, bs, cl.ctypes.data,
                                           len(ctx), K, d, S_out, out.ctypes.data)
    return out


def _roundtrip_passes(kind):
    """Append coded rows with the mutant's layout, gather them back with it."""
    rng = np.random.default_rng(35)
    ctx, table, N, K, d = _paged_case(rng, 4)
    pool = np.zeros((N, K, 4, d), np.float32)
    flat = pool.reshape(-1)
    s = int(ctx.max())
    new = (np.arange(len(ctx) * s * K * d).reshape(len(ctx), s, K, d) + 1).astype(np.float32)
    for b in range(len(ctx)):
        for t in range(int(ctx[b])):
            blk = int(table[b, t // 4])
            for g in range(K):
                row = (blk * 4 + t % 4) * K + g if kind == "head_slot_swapped" else (blk * K + g) * 4 + t % 4
                flat[row * d:(row + 1) * d] = new[b, t, g]
    got = _mutant_gather(kind)(pool, table, ctx, s, np.float32(0))
    return all(np.array_equal(got[b, g, :ctx[b]], new[b, :ctx[b], g]) for b in range(len(ctx)) for g in range(K))


@pytest.mark.parametrize("kind", ["head_slot_swapped", "block_column_off_by_one", "byte_stride"])
def test_planted_paged_mistakes_are_caught(oracle_lib, kind):
    assert _gather_raw_pin_holds(_mutant_gather("none"))
    broken = _byte_stride_gather if kind == "byte_stride" else _mutant_gather(kind)
    assert not _gather_raw_pin_holds(broken)
    if kind == "head_slot_swapped":
        # the swap made consistently on both sides survives a round trip: only
        # the independent indexing above catches it
        assert _roundtrip_passes(kind)


# ---------------------------------------------------------------------------
# planted mistakes: a broken copy of the reference must fail some pin
# ---------------------------------------------------------------------------

def _mutant(kind):
    def ref(q, k, v, q_start, kv_len, causal, scale, window=0):
        B, Sq, H, d = q.shape
        K = k.shape[1]
        G = H // K
        out = np.full(q.shape, np.nan)
        for b in range(B):
            for i in range(Sq):
                qpos = q_start[b] + i
                n = min(kv_len[b], k.shape[2])
                if causal:
                    n = min(n, qpos + (0 if kind == "causal_excludes_self" else 1))
                lo = 0
                if window > 0:
                    lo = max(0, qpos + (0 if kind == "window_off_by_one" else 1) - window)
                if n - lo <= 0:
                    continue
                for h in range(H):
                    g = h % K if kind == "strided_group_map" else h // G
                    sc = 1.0 if kind == "dropped_scale" else scale
                    kk = k[b, g, lo:n]
                    if kind == "transposed_k":
                        kk = k[b, g, lo:n][:, ::-1]
                    s = sc * (kk @ q[b, i, h])
                    p = np.exp(s - s.max())
                    l = p.sum() if kind != "unnormalised" else 1.0
                    out[b, i, h] = (p @ v[b, g, lo:n]) / l
        return out
    return ref


def _pins_pass(ref):
    rng = np.random.default_rng(21)
    B, Sq, H, K, d, Sk = 2, 3, 8, 2, 8, 9
    q, k, v = rand(rng, B, Sq, H, d), rand(rng, B, K, Sk, d), rand(rng, B, K, Sk, d)
    qs, kl = np.array([3, 6], np.int32), np.array([9, 9], np.int32)
    for window in (0, 3):
        got = ref(q, k, v, qs, kl, True, 0.35, window)
        want = sdpa_ref(q, k, v, qs, kl, True, 0.35, window)
        ok = ~np.isnan(want)
        if not np.array_equal(ok, ~np.isnan(got)):
            return False
        if not np.max(np.abs(got[ok] - want[ok])) < 1e-12:
            return False
    return True


@pytest.mark.parametrize("kind", ["strided_group_map", "dropped_scale", "causal_excludes_self",
                                  "transposed_k", "unnormalised", "window_off_by_one"])
def test_planted_mistakes_are_caught(kind):
    assert _pins_pass(_mutant("none"))
    assert not _pins_pass(_mutant(kind))


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache: one fp32 scale per cached row (inference-optimisation
# page §15.5.1: per-token and per-head scales, FP8 E4M3)
# ---------------------------------------------------------------------------

def _torch_e4m3_values() -> np.ndarray:
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e4m3_code_values_match_torch(oracle_lib):
    """Every one of the 256 codes decodes as torch's float8_e4m3fn does."""
    want = _torch_e4m3_values()
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(want))
    fin = np.isfinite(want)
    assert np.array_equal(got[fin], want[fin])
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_rounding_matches_torch(oracle_lib):
    """Nearest value, ties to even: the same codes as torch's fp32 -> float8_e4m3fn cast
    on random values of every magnitude, on every midpoint and on every code value."""
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32) * s for s in (1e-3, 0.05, 1.0, 40.0, 300.0)])
    x = x[np.abs(x) < 448]
    vals = _torch_e4m3_values()
    vals = np.unique(vals[np.isfinite(vals) & (vals >= 0)])
    mids = ((vals[1:] + vals[:-1]) / 2).astype(np.float32)     # exact in fp32: the ties
    x = np.concatenate([x, mids, -mids, vals.astype(np.float32), -vals.astype(np.float32)])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_from_float(v) for v in x], dtype=np.uint8)
    assert np.array_equal(got, want)


def test_e4m3_saturates_at_448(oracle_lib):
    assert oracle.e4m3_from_float(448.0) == 0x7E
    assert oracle.e4m3_from_float(1000.0) == 0x7E
    assert oracle.e4m3_from_float(-1e30) == 0xFE


def _bf16_rows(rng, shape, scale=1.0):
    x = (rng.standard_normal(shape).astype(np.float32) * scale)
    return (((x.view(np.uint32) + 0x7FFF + ((x.view(np.uint32) >> 16) & 1)) >> 16) << 16).view(np.float32)


def test_quantized_row_max_maps_to_448_and_error_is_bounded(oracle_lib):
    """Per row: the largest magnitude becomes +-448, and every element comes back
    within half an E4M3 step (relative 2^-4, or 2^-10 of the scale in the
    subnormal range) of its value."""
    rng = np.random.default_rng(6)
    x = _bf16_rows(rng, (300, 128), 1.0) * rng.lognormal(0, 2, (300, 1)).astype(np.float32)
    codes, scales = oracle.quantize_e4m3_rows(x)
    assert codes.shape == x.shape and scales.shape == (300,)
    amax = np.abs(x).max(axis=1)
    assert np.array_equal(scales, (amax / np.float32(448)).astype(np.float32))
    arg = np.abs(x).argmax(axis=1)
    assert np.all((codes[np.arange(300), arg] & 0x7F) == 0x7E)
    deq = oracle.dequantize_e4m3_rows(codes, scales)
    err = np.abs(deq - x.astype(np.float64))
    bound = np.maximum(np.abs(x) * 2.0 ** -4, scales[:, None].astype(np.float64) * 2.0 ** -10) * (1 + 1e-6)
    assert np.all(err <= bound)


def test_quantization_is_per_row(oracle_lib):
    """Scaling one row by a power of two scales only that row's scale and keeps
    every code (the quotients x / scale do not change)."""
    rng = np.random.default_rng(7)
    x = _bf16_rows(rng, (6, 64))
    c0, s0 = oracle.quantize_e4m3_rows(x)
    y = x.copy()
    y[2] *= np.float32(2.0 ** 5)
    c1, s1 = oracle.quantize_e4m3_rows(y)
    assert np.array_equal(c0, c1)
    assert s1[2] == s0[2] * 2.0 ** 5
    assert np.array_equal(np.delete(s1, 2), np.delete(s0, 2))


def test_zero_row_has_zero_scale_and_codes(oracle_lib):
    x = np.zeros((2, 64), dtype=np.float32)
    x[1, 5] = 3.0
    codes, scales = oracle.quantize_e4m3_rows(x)
    assert scales[0] == 0 and not codes[0].any()
    # the max comes back as 448 * fl32(3 / 448): within one fp32 rounding of 3
    assert abs(oracle.dequantize_e4m3_rows(codes, scales)[1, 5] - 3.0) <= 3.0 * 2.0 ** -24


def test_bf16_bits_input_is_the_same_as_fp32_values(oracle_lib):
    rng = np.random.default_rng(8)
    x = _bf16_rows(rng, (4, 128))
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)
    a = oracle.quantize_e4m3_rows(x)
    b = oracle.quantize_e4m3_rows(bits)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


# ---------------------------------------------------------------------------
# prefill over an FP8 cache: the reading (the new rows quantised as the append
# quantises them, every cached row read as scale * E4M3(code)) pinned to the
# bf16 attention where quantisation is exact, and to per-row scaling
# ---------------------------------------------------------------------------

def _e4m3_exact_rows(rng, shape, scale_exp):
    """Rows whose values are E4M3 values times a power-of-two row scale, each
    row reaching 448 * scale: quantisation returns them unchanged."""
    grid = np.array([oracle.e4m3_value(c) for c in range(0x7F)])       # 0 .. 448, non-negative codes
    grid = grid[np.isfinite(grid)]
    x = rng.choice(grid, size=shape) * rng.choice([-1.0, 1.0], size=shape)
    x[..., 0] = 448.0 * rng.choice([-1.0, 1.0], size=shape[:-1])
    return (x * np.exp2(scale_exp)[..., None]).astype(np.float32)


@pytest.mark.parametrize("paged", [False, True])
def test_fp8_prefill_equals_attention_when_quantisation_is_exact(oracle_lib, paged):
    rng = np.random.default_rng(51)
    B, H, K, d, start, s = 2, 4, 2, 8, 5, 6
    S = start + s
    kp = _e4m3_exact_rows(rng, (B, start, K, d), rng.integers(-9, -3, (B, start, K)))
    vp = _e4m3_exact_rows(rng, (B, start, K, d), rng.integers(-9, -3, (B, start, K)))
    kn = _e4m3_exact_rows(rng, (B, s, K, d), rng.integers(-9, -3, (B, s, K)))
    vn = _e4m3_exact_rows(rng, (B, s, K, d), rng.integers(-9, -3, (B, s, K)))
    q = rand(rng, B, s, H, d)
    table = None
    if paged:
        table, n_pool = np.array([[2, 0, 5], [1, 4, 3]], np.int32), 6
        shape = (n_pool, K, 4, d)
    else:
        shape = (B, K, S, d)
    codes = {n: np.full(shape, 0x7F, np.uint8) for n in "kv"}
    scales = {n: np.full(shape[:-1], np.nan, np.float32) for n in "kv"}
    zero = np.zeros(B, np.int32)
    for n, pre in (("k", kp), ("v", vp)):
        codes[n], scales[n] = oracle.fp8_cache_after_append(codes[n], scales[n], pre, zero, table)
    start_pos = np.full(B, start, np.int32)
    for n, new in (("k", kn), ("v", vn)):
        codes[n], scales[n] = oracle.fp8_cache_after_append(codes[n], scales[n], new, start_pos, table)
    rows = np.array([[b, i, h] for b in range(B) for i in range(s) for h in range(H)], np.int32)
    got = oracle.prefill_fp8_rows(q, codes["k"], scales["k"], codes["v"], scales["v"], start_pos, s, True, 0.3, rows,
                                  block_table=table)
    k_all = np.concatenate([kp, kn], axis=1).transpose(0, 2, 1, 3).astype(np.float64)
    v_all = np.concatenate([vp, vn], axis=1).transpose(0, 2, 1, 3).astype(np.float64)
    want = sdpa_ref(q, k_all, v_all, start_pos, start_pos + s, True, 0.3)
    np.testing.assert_allclose(got, want[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=0, atol=1e-12)


def test_fp8_prefill_scales_with_the_value_rows(oracle_lib):
    """Multiplying every V row by 2^k multiplies the FP8 prefill by 2^k exactly
    (the codes stay, the per-row scales double), while the bf16 rounding of the
    rows before quantisation is exact for powers of two."""
    rng = np.random.default_rng(52)
    B, H, K, d, s = 1, 2, 1, 16, 7
    kn = rng.standard_normal((B, s, K, d)).astype(np.float32)
    vn = rng.standard_normal((B, s, K, d)).astype(np.float32)
    q = rand(rng, B, s, H, d)
    rows = np.array([[0, i, h] for i in range(s) for h in range(H)], np.int32)
    zero = np.zeros(B, np.int32)

    def run(v):
        c = {n: np.zeros((B, K, s, d), np.uint8) for n in "kv"}
        sc = {n: np.zeros((B, K, s), np.float32) for n in "kv"}
        c["k"], sc["k"] = oracle.fp8_cache_after_append(c["k"], sc["k"], kn, zero)
        c["v"], sc["v"] = oracle.fp8_cache_after_append(c["v"], sc["v"], v, zero)
        return oracle.prefill_fp8_rows(q, c["k"], sc["k"], c["v"], sc["v"], zero, s, True, 0.25, rows)
    np.testing.assert_array_equal(run(vn * np.float32(8.0)), 8.0 * run(vn))


# ---------------------------------------------------------------------------
# INT8 KV cache: one fp32 scale per cached row (inference-optimisation page
# §15.5.1 names INT8 beside FP8).  Reading: symmetric, scale = amax / 127,
# code = nearest integer to x * (1 / scale), ties to even, in fp32: the codes
# PyTorch's per-channel qint8 quantiser gives for the same scales.
# ---------------------------------------------------------------------------

def _torch_qint8_codes(x: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """torch.quantize_per_channel along rows with zero points 0 (a library
    routine, independent of the oracle's C code)."""
    x2 = torch.from_numpy(np.ascontiguousarray(x, np.float32).reshape(-1, x.shape[-1]))
    s = torch.from_numpy(np.ascontiguousarray(scales, np.float32).reshape(-1).astype(np.float64))
    q = torch.quantize_per_channel(x2, s, torch.zeros(s.numel(), dtype=torch.int64), 0, torch.qint8)
    return q.int_repr().numpy().reshape(x.shape)


def _int8_tie_rows(rng, n, d):
    """Rows of (integer + 1/2) multiples of a power-of-two step, one element at
    127 steps: every element but the largest is an exact tie."""
    k = rng.integers(-126, 126, size=(n, d)).astype(np.float32) + np.float32(0.5)
    step = np.exp2(rng.integers(-10, 4, size=(n, 1))).astype(np.float32)
    x = (k * step).astype(np.float32)
    x[:, 0] = np.float32(127) * step[:, 0] * rng.choice([-1, 1], size=n).astype(np.float32)
    return x


def test_int8_codes_match_torch_per_channel_quantiser(oracle_lib):
    """Random rows over many magnitudes and rows of exact ties: the oracle's
    codes are the ones torch.quantize_per_channel (qint8, zero point 0) gives
    for the same per-row scales."""
    rng = np.random.default_rng(61)
    x = _bf16_rows(rng, (3000, 128), 1.0) * rng.lognormal(0, 3, (3000, 1)).astype(np.float32)
    codes, scales = oracle.quantize_i8_rows(x)
    assert codes.dtype == np.int8 and scales.dtype == np.float32
    assert np.array_equal(codes, _torch_qint8_codes(x, scales))
    t = _int8_tie_rows(rng, 2000, 64)
    tc, ts = oracle.quantize_i8_rows(t)
    assert np.array_equal(tc, _torch_qint8_codes(t, ts))
    # the ties really are ties, resolved to the even neighbour
    assert np.all(np.abs(tc[:, 1:]) % 2 == 0)


def test_int8_row_max_maps_to_127_and_error_is_bounded(oracle_lib):
    """Per row: the largest magnitude becomes +-127, scale * 127 is the row's
    largest magnitude to fp32 rounding, and every element comes back within
    half a step (scale / 2) of its value."""
    rng = np.random.default_rng(62)
    x = _bf16_rows(rng, (400, 128), 1.0) * rng.lognormal(0, 2, (400, 1)).astype(np.float32)
    codes, scales = oracle.quantize_i8_rows(x)
    amax = np.abs(x).max(axis=1).astype(np.float64)
    arg = np.abs(x).argmax(axis=1)
    assert np.all(np.abs(codes[np.arange(400), arg].astype(np.int32)) == 127)
    assert np.all(np.abs(codes.astype(np.int32)) <= 127)
    assert np.all(np.abs(scales.astype(np.float64) * 127 - amax) <= amax * 2.0 ** -23)
    err = np.abs(oracle.dequantize_i8_rows(codes, scales) - x.astype(np.float64))
    assert np.all(err <= scales[:, None].astype(np.float64) * (0.5 + 2.0 ** -16))


def test_int8_quantization_is_per_row(oracle_lib):
    """Scaling one row by a power of two scales only that row's scale and keeps
    every code; an all-zero row has scale 0 and zero codes."""
    rng = np.random.default_rng(63)
    x = _bf16_rows(rng, (6, 64))
    x[4] = 0.0
    c0, s0 = oracle.quantize_i8_rows(x)
    y = x.copy()
    y[2] *= np.float32(2.0 ** -7)
    c1, s1 = oracle.quantize_i8_rows(y)
    assert np.array_equal(c0, c1)
    assert s1[2] == s0[2] * 2.0 ** -7
    assert np.array_equal(np.delete(s1, 2), np.delete(s0, 2))
    assert s0[4] == 0 and not c0[4].any()
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)   # bf16 bits in, the same rows
    cb, sb = oracle.quantize_i8_rows(bits)
    assert np.array_equal(cb, c0) and np.array_equal(sb, s0)


def _i8_exact_rows(rng, shape, scale_exp):
    """Rows of integers in [-127, 127] times a power-of-two row scale, each row
    reaching 127 * scale: quantisation returns them unchanged."""
    x = rng.integers(-127, 128, size=shape).astype(np.float64)
    x[..., 0] = 127.0 * rng.choice([-1.0, 1.0], size=shape[:-1])
    return (x * np.exp2(scale_exp)[..., None]).astype(np.float32)


@pytest.mark.parametrize("paged", [False, True])
def test_int8_prefill_equals_attention_when_quantisation_is_exact(oracle_lib, paged):
    rng = np.random.default_rng(64)
    B, H, K, d, start, s = 2, 4, 2, 8, 5, 6
    S = start + s
    kp = _i8_exact_rows(rng, (B, start, K, d), rng.integers(-12, -6, (B, start, K)))
    vp = _i8_exact_rows(rng, (B, start, K, d), rng.integers(-12, -6, (B, start, K)))
    kn = _i8_exact_rows(rng, (B, s, K, d), rng.integers(-12, -6, (B, s, K)))
    vn = _i8_exact_rows(rng, (B, s, K, d), rng.integers(-12, -6, (B, s, K)))
    q = rand(rng, B, s, H, d)
    table = None
    if paged:
        table, n_pool = np.array([[2, 0, 5], [1, 4, 3]], np.int32), 6
        shape = (n_pool, K, 4, d)
    else:
        shape = (B, K, S, d)
    codes = {n: np.full(shape, 0x7F, np.int8) for n in "kv"}
    scales = {n: np.full(shape[:-1], np.nan, np.float32) for n in "kv"}
    zero = np.zeros(B, np.int32)
    for n, pre in (("k", kp), ("v", vp)):
        codes[n], scales[n] = oracle.fp8_cache_after_append(codes[n], scales[n], pre, zero, table, codec="int8")
    start_pos = np.full(B, start, np.int32)
    for n, new in (("k", kn), ("v", vn)):
        codes[n], scales[n] = oracle.fp8_cache_after_append(codes[n], scales[n], new, start_pos, table, codec="int8")
    assert codes["k"].dtype == np.int8
    rows = np.array([[b, i, h] for b in range(B) for i in range(s) for h in range(H)], np.int32)
    got = oracle.prefill_fp8_rows(q, codes["k"], scales["k"], codes["v"], scales["v"], start_pos, s, True, 0.3, rows,
                                  block_table=table, codec="int8")
    k_all = np.concatenate([kp, kn], axis=1).transpose(0, 2, 1, 3).astype(np.float64)
    v_all = np.concatenate([vp, vn], axis=1).transpose(0, 2, 1, 3).astype(np.float64)
    want = sdpa_ref(q, k_all, v_all, start_pos, start_pos + s, True, 0.3)
    np.testing.assert_allclose(got, want[rows[:, 0], rows[:, 1], rows[:, 2]], rtol=0, atol=1e-12)


@pytest.mark.parametrize("kind", ["truncate", "scale_128", "divide_by_reciprocal_of_128", "round_half_away"])
def test_planted_int8_mistakes_are_caught(oracle_lib, kind):
    """A plausible wrong INT8 quantiser, written out on the CPU, fails the
    torch pin above on the same rows."""
    rng = np.random.default_rng(65)
    x = np.concatenate([_bf16_rows(rng, (500, 64)) * rng.lognormal(0, 2, (500, 1)).astype(np.float32),
                        _int8_tie_rows(rng, 500, 64)])
    amax = np.abs(x).max(axis=1).astype(np.float32)
    if kind == "scale_128":
        scale = (amax / np.float32(128)).astype(np.float32)
    else:
        scale = (amax / np.float32(127)).astype(np.float32)
    inv = (np.float32(1) / scale).astype(np.float32)
    qf = (x * inv[:, None]).astype(np.float32)
    if kind == "truncate":
        codes = np.trunc(qf)
    elif kind == "round_half_away":
        codes = np.sign(qf) * np.floor(np.abs(qf) + np.float32(0.5))
    elif kind == "divide_by_reciprocal_of_128":
        codes = np.rint((x * (np.float32(1) / (amax / np.float32(128)))[:, None]).astype(np.float32))
    else:
        codes = np.rint(qf)
    codes = np.clip(codes, -127, 127).astype(np.int8)
    ok_scale = (amax / np.float32(127)).astype(np.float32)
    caught = not np.array_equal(codes, _torch_qint8_codes(x, ok_scale)) or not np.array_equal(scale, ok_scale)
    assert caught, kind
