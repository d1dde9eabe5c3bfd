"""GPU parity: libgqa (through the C ABI) against the fp64 CPU oracle on the
same seeded bits.

Tolerances: bf16 inputs with fp32 accumulation, max abs error <= 2e-2; the
fp32 path <= 1e-5; cache appends bit-exact.  Small cases compare every
output; the full-size workloads, in the launch configuration the bench
times, compare sampled rows that the oracle evaluates one by one.  Unused
cache slots hold NaN, so a stray read shows up as a non-finite output."""
import numpy as np
import pytest
import torch

import oracle
from grouped_query_attention_gqa_amd import binding
from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import (BF16_TOL, F32_TOL, DecodeRun, PrefillRun, as_f64, check_close, from_dev, gpu_rows,
                        oracle_decode_rows, oracle_prefill_rows, requires_gpu, say, to_dev)

pytestmark = [pytest.mark.gpu, requires_gpu]


def _tol(dtype):
    return BF16_TOL if dtype == "bf16" else F32_TOL


# ---------------------------------------------------------------------------
# gqa_kv_append: bit-exact against the oracle's indexed copy
# ---------------------------------------------------------------------------

def _random_rows(rng, shape, dtype):
    if dtype == "bf16":
        return W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    return rng.standard_normal(shape, dtype=np.float32)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_append_contiguous_bit_exact(dtype, d):
    rng = np.random.default_rng(100 + d)
    B, K, S, s_new = 3, 4, 160, 37
    start = np.array([0, 5, 140], np.int32)      # the last one runs past S: those rows are dropped
    cache = np.full((B, K, S, d), W.sentinel(dtype, "nan"), dtype=W.storage_dtype(dtype))
    kn, vn = _random_rows(rng, (B, s_new, K, d), dtype), _random_rows(rng, (B, s_new, K, d), dtype)
    say("append contiguous", dtype, d)
    kc, vc = to_dev(cache), to_dev(cache)
    c = binding.KVCache(kc, vc)
    binding.gqa_kv_append(c, to_dev(kn), to_dev(vn), to_dev(start))
    torch.cuda.synchronize()
    want_k, want_v = cache.copy(), cache.copy()
    oracle.kv_append(want_k, kn, start)
    oracle.kv_append(want_v, vn, start)
    assert from_dev(kc).tobytes() == want_k.tobytes()
    assert from_dev(vc).tobytes() == want_v.tobytes()


@pytest.mark.parametrize("s_new", [1, 29])
def test_append_paged_bit_exact(s_new):
    rng = np.random.default_rng(7 + s_new)
    dtype, B, K, d, bs = "bf16", 4, 8, 128, 16
    ctx_cap = np.array([40, 16, 300, 77], np.int32)
    table, n_pool = W.deal_blocks(rng, ctx_cap, bs, slack_blocks=3)
    start = np.array([3, 0, 250, 77 - s_new], np.int32)
    pool = np.full((n_pool, K, bs, d), W.sentinel(dtype, "nan"), dtype=np.uint16)
    kn, vn = _random_rows(rng, (B, s_new, K, d), dtype), _random_rows(rng, (B, s_new, K, d), dtype)
    say("append paged", s_new)
    kp, vp = to_dev(pool), to_dev(pool)
    c = binding.KVCache(kp, vp, to_dev(table))
    binding.gqa_kv_append(c, to_dev(kn), to_dev(vn), to_dev(start))
    torch.cuda.synchronize()
    want_k, want_v = pool.copy(), pool.copy()
    oracle.kv_append_paged(want_k, kn, start, table)
    oracle.kv_append_paged(want_v, vn, start, table)
    assert from_dev(kp).tobytes() == want_k.tobytes()
    assert from_dev(vp).tobytes() == want_v.tobytes()


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

def _decode_case(inp, what, seqs=None, heads=None, window=0):
    say("decode", what, inp.wl.B, inp.wl.H, inp.wl.K, inp.wl.d, "ctx max", int(inp.ctx.max()), "window", window)
    run = DecodeRun(inp)
    out = from_dev(run.run(window=window))
    rows, want = oracle_decode_rows(inp, seqs, heads, window)
    got = gpu_rows(out, rows, inp.wl.dtype)
    return check_close(got, want, _tol(inp.wl.dtype), what)


def test_tiny_decode_f32():
    inp = W.make_decode(W.WORKLOADS["tiny_decode_f32"])
    _decode_case(inp, "tiny fp32 decode")


@pytest.mark.parametrize("H,K", [(32, 8), (64, 8), (64, 64), (64, 1), (24, 8), (16, 16), (8, 2)])
@pytest.mark.parametrize("d", [128, 64])
def test_decode_bf16_ragged(H, K, d):
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=4, H=H, K=K, d=d, ctx=("uniform", 1, 700))
    inp = W.make_decode(wl, ctx_override=[1, 63, 700, 129])
    _decode_case(inp, f"bf16 decode H={H} K={K} d={d}")


@pytest.mark.parametrize("H,K,d", [(8, 2, 64), (64, 8, 128), (32, 32, 64)])
def test_decode_f32_multi_split(H, K, d):
    wl = W.WORKLOADS["tiny_decode_f32"].replace(B=3, H=H, K=K, d=d, ctx=("uniform", 1, 1500))
    inp = W.make_decode(wl, ctx_override=[1500, 2, 333])
    _decode_case(inp, f"fp32 decode H={H} K={K} d={d}")


@pytest.mark.parametrize("bs", [1, 4, 8, 32, 64, 256])
def test_decode_paged_block_sizes(bs):
    wl = W.WORKLOADS["paged_long_decode"].replace(B=3, ctx=("loguniform", 17, 1500), block_size=bs)
    inp = W.make_decode(wl)
    _decode_case(inp, f"paged bf16 decode, {bs}-token blocks")


def test_decode_paged_small():
    wl = W.WORKLOADS["paged_long_decode"].replace(B=6, ctx=("loguniform", 17, 3000))
    inp = W.make_decode(wl)
    _decode_case(inp, "paged bf16 decode")


@pytest.mark.parametrize("B,ctx", [(1, 1), (1, 63), (1, 64), (1, 65), (2, 16448), (3, 200000 // 3), (300, 40)])
def test_decode_slices_cut_items_anywhere(B, ctx):
    """Rows shorter than a tile, exactly a tile, and long rows cut by many workgroup slices."""
    wl = W.WORKLOADS["llama2_70b_decode"].replace(B=B, ctx=("fixed", ctx))
    inp = W.make_decode(wl)
    seqs = sorted({0, B - 1, B // 2})
    _decode_case(inp, f"decode B={B} ctx={ctx}", seqs=seqs)


def test_decode_more_rows_than_one_launch():
    """B above the 512 rows one launch handles: the rows run in consecutive launches."""
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=1100, ctx=("uniform", 1, 300))
    inp = W.make_decode(wl)
    _decode_case(inp, "decode B=1100", seqs=[0, 1, 511, 512, 513, 1023, 1024, 1099])


def test_decode_workspace_reused_across_layouts():
    """One workspace serves calls whose split layouts overlap each other's bytes."""
    a = W.make_decode(W.WORKLOADS["llama2_70b_decode"].replace(B=2, ctx=("fixed", 3000)))
    b = W.make_decode(W.WORKLOADS["llama3_8b_decode"].replace(B=8, ctx=("uniform", 300, 1300)))
    c = W.make_decode(W.WORKLOADS["llama2_70b_decode_mqa"].replace(B=3, ctx=("uniform", 900, 5000)))
    need = max(binding.gqa_decode_workspace_bytes(i.wl.B, i.wl.H, i.wl.K, i.wl.d, int(i.ctx.max())) for i in (a, b, c))
    ws = torch.zeros(need, dtype=torch.uint8, device="cuda")
    for inp, what in ((a, "A"), (b, "B"), (c, "C"), (a, "A again"), (b, "B again")):
        say("workspace reuse", what)
        out = from_dev(DecodeRun(inp).run(workspace=ws))
        rows, want = oracle_decode_rows(inp)
        check_close(gpu_rows(out, rows, "bf16"), want, BF16_TOL, f"workspace reuse {what}")


# full-size workloads, sampled rows -------------------------------------------

def _sample_seqs(inp, n=6):
    order = np.argsort(inp.ctx, kind="stable")
    pick = {int(order[0]), int(order[-1]), int(order[len(order) // 2])}
    rng = np.random.default_rng(5)
    pick |= set(int(x) for x in rng.choice(inp.wl.B, size=min(n, inp.wl.B), replace=False))
    return sorted(pick)[:n + 3]


@pytest.mark.parametrize("name", ["llama3_8b_decode", "llama2_70b_decode", "llama2_70b_decode_mqa",
                                  "llama2_70b_decode_mha", "paged_long_decode"])
def test_full_size_decode_sampled(name):
    wl = W.WORKLOADS[name]
    inp = W.make_decode(wl)
    seqs = _sample_seqs(inp)
    heads = sorted({0, 1, wl.G - 1, wl.G, wl.H // 2, wl.H - 1} & set(range(wl.H)))
    _decode_case(inp, f"{name} (sampled)", seqs, heads)


# ---------------------------------------------------------------------------
# prefill
# ---------------------------------------------------------------------------

def _all_rows(B, s, H):
    return np.array([[b, i, h] for b in range(B) for i in range(s) for h in range(H)], np.int32)


def _prefill_case(inp, what, rows=None, causal=True, window=0, **kw):
    wl = inp.wl
    say("prefill", what, wl.B, wl.s, wl.H, wl.K, wl.d, "causal", causal, "window", window)
    run = PrefillRun(inp, **kw)
    out = from_dev(run.run(causal=causal, window=window))
    run.check_cache(what)   # the bytes the oracle's append writes
    rows = _all_rows(wl.B, wl.s, wl.H) if rows is None else rows
    want = oracle_prefill_rows(inp, rows, causal=causal, prior=kw.get("prior"), window=window)
    return check_close(gpu_rows(out, rows, wl.dtype), want, _tol(wl.dtype), what), run


def test_tiny_prefill_f32():
    _prefill_case(W.make_prefill(W.WORKLOADS["tiny_prefill_f32"]), "tiny fp32 prefill")


@pytest.mark.parametrize("H,K", [(32, 8), (8, 8), (64, 1), (24, 8), (64, 8), (16, 2)])
@pytest.mark.parametrize("d", [128, 64])
def test_prefill_bf16_ragged(H, K, d):
    wl = W.WORKLOADS["causal_prefill_4k"].replace(B=2, s=200, H=H, K=K, d=d)
    _prefill_case(W.make_prefill(wl), f"bf16 prefill H={H} K={K} d={d}")


def test_prefill_bf16_not_causal():
    wl = W.WORKLOADS["causal_prefill_4k"].replace(B=2, s=150)
    _prefill_case(W.make_prefill(wl), "bf16 prefill, not causal", causal=False)


def test_prefill_f32_not_causal():
    wl = W.WORKLOADS["tiny_prefill_f32"].replace(B=2, s=70)
    _prefill_case(W.make_prefill(wl), "fp32 prefill, not causal", causal=False)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_continues_cached_prefix(dtype):
    """start_pos > 0: the new rows attend to the cached prefix and to themselves."""
    base = W.WORKLOADS["causal_prefill_4k"] if dtype == "bf16" else W.WORKLOADS["tiny_prefill_f32"]
    wl = base.replace(B=2, s=96, H=16, K=4, d=128 if dtype == "bf16" else 64)
    inp = W.make_prefill(wl)
    P = 173
    rng = np.random.default_rng(3)
    prior = (_random_rows(rng, (wl.B, P, wl.K, wl.d), dtype), _random_rows(rng, (wl.B, P, wl.K, wl.d), dtype))
    inp = W.PrefillInputs(wl, np.full(wl.B, P, np.int32), inp.q, inp.k_new, inp.v_new)
    _prefill_case(inp, f"{dtype} prefill after a {P}-token prefix", prior=prior)


def test_prefill_paged_cache():
    wl = W.WORKLOADS["causal_prefill_4k"].replace(B=3, s=130, H=32, K=8)
    rng = np.random.default_rng(11)
    table, n_pool = W.deal_blocks(rng, np.full(wl.B, wl.s, np.int32), wl.block_size, slack_blocks=5)
    (worst, run) = _prefill_case(W.make_prefill(wl), "bf16 prefill into a paged cache",
                                 paged_blocks=(table, n_pool))
    # the cache bytes equal what the oracle's paged append writes
    inp = run.inp
    pool = np.full((n_pool, wl.K, wl.block_size, wl.d), W.sentinel("bf16", "nan"), dtype=np.uint16)
    oracle.kv_append_paged(pool, inp.k_new, inp.start_pos, table)
    assert from_dev(run.k).tobytes() == pool.tobytes()


def test_full_size_prefill_sampled():
    wl = W.WORKLOADS["causal_prefill_4k"]
    inp = W.make_prefill(wl)
    rng = np.random.default_rng(17)
    pos = sorted({0, 1, 31, 32, 63, 64, 127, 128, 2047, 4095} | set(int(x) for x in rng.integers(0, wl.s, 6)))
    rows = np.array([[b, i, h] for b in range(wl.B) for i in pos for h in (0, 3, 4, 17, 31)], np.int32)
    worst, run = _prefill_case(inp, "causal_prefill_4k (sampled)", rows=rows)
    # the cache the prefill wrote equals the oracle's append
    cache = np.full((wl.B, wl.K, wl.s, wl.d), W.sentinel("bf16", "nan"), dtype=np.uint16)
    oracle.kv_append(cache, inp.k_new, inp.start_pos)
    assert from_dev(run.k).tobytes() == cache.tobytes()


def test_full_size_chunked_prefill_sampled():
    """The chunked paged prefill at the size the bench times: 512 new tokens
    after a 3584-token prefix already in a shuffled 16-token paged cache."""
    wl = W.WORKLOADS["chunked_prefill_paged"]
    inp = W.make_prefill(wl)
    rng = np.random.default_rng(19)
    P = wl.start
    prior = (_random_rows(rng, (wl.B, P, wl.K, wl.d), "bf16"), _random_rows(rng, (wl.B, P, wl.K, wl.d), "bf16"))
    table, n_pool = W.deal_blocks(rng, np.full(wl.B, P + wl.s, np.int32), wl.block_size)
    pos = sorted({0, 1, 15, 16, 63, 64, 255, 511} | set(int(x) for x in rng.integers(0, wl.s, 4)))
    rows = np.array([[b, i, h] for b in range(wl.B) for i in pos for h in (0, 3, 4, 17, 31)], np.int32)
    _prefill_case(inp, "chunked_prefill_paged (sampled)", rows=rows, paged_blocks=(table, n_pool), prior=prior)
