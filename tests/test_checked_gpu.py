"""Checked mode (GQA_CHECK=1) and the decode's split count on the GPU.

With GQA_CHECK=1 the host copies the device-resident integers back (context
lengths, start positions, block ids), validates them and returns
GQA_ERR_DEVICE_ARG before launching anything: the outputs and the cache keep
their bytes.  Entries of blocks that lie wholly below a sliding window are
never read, so they may be stale and the checked call still runs.

GQA_DECODE_WGS=n fixes how many workgroups a decode splits the keys over.
Flash-decoding's split and merge are exact rewrites of the softmax
(inference-optimisation page §10.2), so every split count must match the
oracle, and each one must be deterministic.
"""
import numpy as np
import pytest
import torch

from grouped_query_attention_gqa_amd import binding
from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import (BF16_TOL, F32_TOL, DecodeRun, as_f64, check_close, from_dev, gpu_rows, oracle_decode_rows,
                        requires_gpu, say, to_dev)

pytestmark = [pytest.mark.gpu, requires_gpu]

BF16 = lambda x: W.f32_to_bf16_bits(np.asarray(x, np.float32))


@pytest.fixture
def checked(monkeypatch):
    monkeypatch.setenv("GQA_CHECK", "1")


def _rejected(fn):
    with pytest.raises(binding.GqaError) as e:
        fn()
    assert e.value.status == binding.GQA_ERR_DEVICE_ARG, e.value


def _sentinel_like(t):
    return torch.full_like(t, 7.0)


def test_checked_decode_rejects_bad_context_lengths(checked):
    inp = W.make_decode(W.WORKLOADS["llama3_8b_decode"].replace(B=3, ctx=("uniform", 10, 300)),
                        ctx_override=[50, 300, 9])
    run = DecodeRun(inp)
    out = _sentinel_like(run.q)
    for bad, max_ctx in (([50, 0, 9], 300), ([50, 301, 9], 300), ([50, -4, 9], 300)):
        say("checked decode ctx", bad)
        ctx = to_dev(np.array(bad, np.int32))
        _rejected(lambda: binding.gqa_decode(run.q, run.cache, ctx, max_ctx, out=out))
    # a length past the cache capacity (S_max = 300), even under a larger max_ctx
    ctx = to_dev(np.array([50, 301, 9], np.int32))
    _rejected(lambda: binding.gqa_decode(run.q, run.cache, ctx, 400, out=out))
    kn, vn = (to_dev(x) for x in inp.new_token_rows())
    k0, v0 = from_dev(run.k).copy(), from_dev(run.v).copy()
    _rejected(lambda: binding.gqa_decode_step(run.q, kn, vn, run.cache, to_dev(np.array([50, 0, 9], np.int32)), 300,
                                              out=out))
    torch.cuda.synchronize()
    assert (out == 7.0).all()
    assert from_dev(run.k).tobytes() == k0.tobytes() and from_dev(run.v).tobytes() == v0.tobytes()
    # the valid call runs and equals the unchecked result
    got = from_dev(run.run(out=out))
    assert np.isfinite(as_f64(got, "bf16")).all()


def test_checked_decode_multi_rejects_short_context(checked):
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=2, ctx=("uniform", 10, 300))
    inp = W.make_decode(wl, ctx_override=[3, 200])
    run = DecodeRun(inp)
    q = to_dev(BF16(np.random.default_rng(0).standard_normal((2, 4, wl.H, wl.d))))
    out = _sentinel_like(q)
    say("checked decode multi")
    _rejected(lambda: binding.gqa_decode_multi(q, run.cache, run.ctx, 200, out=out))   # ctx 3 < s = 4
    torch.cuda.synchronize()
    assert (out == 7.0).all()


def test_checked_paged_decode_block_ids(checked):
    wl = W.WORKLOADS["paged_long_decode"].replace(B=3, ctx=("uniform", 100, 900))
    inp = W.make_decode(wl)
    run = DecodeRun(inp)
    good = run.run()
    n_pool = inp.k.shape[0]
    for bad_id in (n_pool, -1, 1 << 30):
        table = inp.block_table.copy()
        table[1, int(inp.ctx[1] - 1) // 16] = bad_id      # the block of the newest token
        cache = binding.KVCache(run.k, run.v, to_dev(table))
        out = _sentinel_like(run.q)
        say("checked paged decode id", bad_id)
        _rejected(lambda: binding.gqa_decode(run.q, cache, run.ctx, run.max_ctx, out=out))
        torch.cuda.synchronize()
        assert (out == 7.0).all()
    # a window of 64: blocks wholly below every window may hold stale ids
    win = 64
    want = run.run(window=win)
    table = inp.block_table.copy()
    for b in range(wl.B):
        lo = max(0, int(inp.ctx[b]) - win)
        table[b, :lo // 16] = [-1, n_pool, 1 << 30][b]
    cache = binding.KVCache(run.k, run.v, to_dev(table))
    say("checked paged decode, stale ids below the window")
    out = binding.gqa_decode(run.q, cache, run.ctx, run.max_ctx, window=win)
    torch.cuda.synchronize()
    assert from_dev(out).tobytes() == from_dev(want).tobytes()
    # one id inside the window out of range: rejected
    table[0, (int(inp.ctx[0]) - 1) // 16] = n_pool + 3
    cache = binding.KVCache(run.k, run.v, to_dev(table))
    _rejected(lambda: binding.gqa_decode(run.q, cache, run.ctx, run.max_ctx, window=win))
    del good


def test_checked_prefill_and_append(checked):
    wl = W.WORKLOADS["causal_prefill_4k"].replace(B=2, s=40)
    inp = W.make_prefill(wl)
    q, kn, vn = to_dev(inp.q), to_dev(inp.k_new), to_dev(inp.v_new)
    S = 100
    k = torch.zeros(wl.B, wl.K, S, wl.d, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    cache = binding.KVCache(k, v)
    out = _sentinel_like(q)
    for bad in ([0, -1], [0, 61]):          # negative; 61 + 40 > S_max = 100
        say("checked prefill start", bad)
        sp = to_dev(np.array(bad, np.int32))
        _rejected(lambda: binding.gqa_prefill(q, kn, vn, cache, sp, out=out))
        _rejected(lambda: binding.gqa_kv_append(cache, kn, vn, sp))
    torch.cuda.synchronize()
    assert (out == 7.0).all() and (k == 0).all() and (v == 0).all()
    # paged: a bad id in the prefix is rejected; with a window, ids wholly below
    # the oldest row's window may be stale
    bs, start = 16, 60
    table, n_pool = W.deal_blocks(np.random.default_rng(3), np.full(wl.B, start + wl.s, np.int32), bs)
    pk = torch.zeros(n_pool, wl.K, bs, wl.d, dtype=torch.bfloat16, device="cuda")
    pv = torch.zeros_like(pk)
    sp = to_dev(np.full(wl.B, start, np.int32))
    bad = table.copy()
    bad[1, 0] = n_pool
    pc = binding.KVCache(pk, pv, to_dev(bad))
    say("checked paged prefill bad id")
    _rejected(lambda: binding.gqa_prefill(q, kn, vn, pc, sp, out=out))
    stale = table.copy()
    stale[:, 0] = [-1, n_pool]      # keys 0-15: below every window of 40 (oldest row at 60 sees 21..)
    pc = binding.KVCache(pk, pv, to_dev(stale))
    say("checked paged prefill, stale ids below the window")
    got = binding.gqa_prefill(q, kn, vn, pc, sp, window=40)
    torch.cuda.synchronize()
    assert np.isfinite(as_f64(from_dev(got), "bf16")).all()


# ---------------------------------------------------------------------------
# the split count
# ---------------------------------------------------------------------------

SPLIT_CASES = {
    # name: (workload, tolerance) -- one case per decode kernel
    "mfma_g4": (W.WORKLOADS["llama3_8b_decode"].replace(B=5, ctx=("uniform", 1, 3000)), BF16_TOL),
    "mfma_g64_paged": (W.WORKLOADS["paged_long_decode"].replace(B=3, H=64, K=1, ctx=("loguniform", 30, 4000)),
                       BF16_TOL),
    "mfma_g32": (W.WORKLOADS["llama3_8b_decode"].replace(B=3, H=64, K=2, ctx=("uniform", 1, 2000)), BF16_TOL),
    "mfma_d64": (W.WORKLOADS["llama3_8b_decode"].replace(B=4, d=64, ctx=("uniform", 1, 2000)), BF16_TOL),
    "mfma_d64_g16": (W.WORKLOADS["llama3_8b_decode"].replace(B=3, d=64, H=32, K=2, ctx=("uniform", 1, 1500)),
                     BF16_TOL),
    # blocks of 4 tokens: the stream kernel's bf16 path
    "stream_bf16_blocks4": (W.WORKLOADS["paged_long_decode"].replace(B=3, H=32, K=8, ctx=("loguniform", 30, 1500),
                                                                     block_size=4), BF16_TOL),
    "stream_f32": (W.WORKLOADS["tiny_decode_f32"].replace(B=3, ctx=("uniform", 1, 700)), F32_TOL),
}


@pytest.mark.parametrize("wgs", [1, 7, 64, 512])
@pytest.mark.parametrize("case", sorted(SPLIT_CASES))
def test_decode_every_split_count_matches_oracle(monkeypatch, case, wgs):
    wl, tol = SPLIT_CASES[case]
    inp = W.make_decode(wl)
    run = DecodeRun(inp)
    monkeypatch.setenv("GQA_DECODE_WGS", str(wgs))
    say("split count", case, wgs)
    a = from_dev(run.run())
    b = from_dev(run.run())
    assert a.tobytes() == b.tobytes(), "not deterministic at a fixed split count"
    rows, want = oracle_decode_rows(inp)
    check_close(gpu_rows(a, rows, wl.dtype), want, tol, f"{case} with {wgs} workgroups")


@pytest.mark.parametrize("wgs", [1, 7, 64, 512])
def test_decode_split_count_keeps_window_coverage_exact(monkeypatch, wgs):
    """The exact 128-token window test at each split count: the slices cut the
    items anywhere, and every cached token is still counted once."""
    wl = W.WORKLOADS["paged_long_decode"].replace(B=4)
    ctx = np.array([129, 1000, 3001, 2051], np.int32)
    rng = np.random.default_rng(wgs)
    inp = W.make_decode(wl, ctx_override=ctx)
    u = rng.choice([-1.0, 1.0], size=(wl.B, wl.K, wl.d)).astype(np.float32)
    for b in range(wl.B):
        n = int(ctx[b])
        t = np.arange(n)
        blk, slot = inp.block_table[b, t // 16].astype(np.int64), t % 16
        for g in range(wl.K):
            inp.q[b, 0, g * wl.G:(g + 1) * wl.G] = BF16(u[b, g])
            lo = int(rng.integers(0, n - 128 + 1))
            inside = (t >= lo) & (t < lo + 128)
            inp.k[blk, g, slot] = BF16(np.where(inside[:, None], 2.5 * u[b, g][None, :], 0.0))
            rows = np.zeros((n, wl.d), np.float32)
            rows[t, t % wl.d] = 1.0
            inp.v[blk, g, slot] = BF16(rows)
    monkeypatch.setenv("GQA_DECODE_WGS", str(wgs))
    say("split count window", wgs)
    out = as_f64(from_dev(DecodeRun(inp).run()), "bf16")
    assert np.array_equal(out, np.full(out.shape, 1.0 / 128.0))
