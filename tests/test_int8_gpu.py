"""INT8 KV cache with one fp32 scale per cached row (inference-optimisation
page §15.5-§15.5.1 names INT8 beside FP8), through the C ABI, against the
oracle.

* The quantising append must give the oracle's codes and scales bit for bit
  (both decide in fp32: scale = amax / 127, code = nearest-even of
  x * (1 / scale)).
* Decode and prefill on an INT8 cache must match the fp64 oracle attention
  over the dequantised values (scale * code) within the bf16 tolerance.
* Structured inputs whose rows are integers times a power-of-two scale make
  the INT8 round trip exact, so a wrong block, slot or scale changes a bit.
Unused cache slots hold code -128 (never written by the quantiser) and NaN
scales, so a read of one shows."""
import numpy as np
import pytest
import torch

import oracle
from grouped_query_attention_gqa_amd import binding
from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import BF16_TOL, as_f64, check_close, from_dev, say, to_dev
from test_fp8_gpu import (_check_fp8_prefill, _decode_case, _f8_cache, dequant, f8_dev, f8_host, oracle_rows_f8,
                          quantized_inputs)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LLAMA3 = W.WORKLOADS["llama3_8b_decode"]
BF16 = lambda x: W.f32_to_bf16_bits(np.asarray(x, np.float32))


def _append_case(paged: bool):
    rng = np.random.default_rng(21 + paged)
    B, s_new, K, d = (3, 5, 8, 128) if not paged else (2, 20, 8, 128)
    kn = W.f32_to_bf16_bits(rng.standard_normal((B, s_new, K, d)).astype(np.float32)
                            * rng.lognormal(0, 2, (B, s_new, K, 1)).astype(np.float32))
    vn = W.f32_to_bf16_bits(rng.standard_normal((B, s_new, K, d)).astype(np.float32) * 7)
    kn[0, 0, 0] = 0                                                # an all-zero row
    kn[1, 2, 3] = W.f32_to_bf16_bits(np.float32([1e-3] * d))
    kn[1, 2, 3, 7] = W.f32_to_bf16_bits(np.float32([-3.0e4]))[0]   # one large negative value
    # rows of exact ties: (integer + 1/2) steps of a power of two, one element at 127 steps
    t = rng.integers(-126, 126, size=(d,)).astype(np.float32) + np.float32(0.5)
    t[0] = 127.0
    vn[0, 1, 2] = W.f32_to_bf16_bits(t * np.float32(2.0 ** -6))
    if paged:
        bs, N = 16, 6
        table = np.array([[3, 0, 5], [1, 4, 2]], dtype=np.int32)
        start = np.array([9, 0], dtype=np.int32)
        shape = (N, K, bs, d)
    else:
        S = 40
        table = None
        start = np.array([0, 17, 37], dtype=np.int32)   # the last one runs past S_max: those rows are skipped
        shape = (B, K, S, d)
    codes0 = np.full(shape, 0xAB, dtype=np.uint8)
    scales0 = np.full(shape[:-1], np.nan, dtype=np.float32)
    kc, vc, ksc, vsc = f8_dev(codes0, "int8"), f8_dev(codes0, "int8"), to_dev(scales0), to_dev(scales0)
    cache = binding.KVCache(kc, vc, None if table is None else to_dev(table), k_scale=ksc, v_scale=vsc)
    say("int8 append", f"paged={paged}")
    binding.gqa_kv_append(cache, to_dev(kn), to_dev(vn), to_dev(start))
    torch.cuda.synchronize()
    for name, new, codes_d, sc_d in (("k", kn, kc, ksc), ("v", vn, vc, vsc)):
        want_c, want_s = codes0.copy(), scales0.copy()
        qc, qs = oracle.quantize_i8_rows(new)
        qc = qc.view(np.uint8)
        for b in range(B):
            for t_ in range(s_new):
                pos = int(start[b]) + t_
                if table is None:
                    if pos < shape[2]:
                        want_c[b, :, pos] = qc[b, t_]
                        want_s[b, :, pos] = qs[b, t_]
                else:
                    blk = table[b, pos // shape[2]]
                    want_c[blk, :, pos % shape[2]] = qc[b, t_]
                    want_s[blk, :, pos % shape[2]] = qs[b, t_]
        assert np.array_equal(f8_host(codes_d), want_c), f"{name} codes differ"
        assert sc_d.cpu().numpy().view(np.uint32).tobytes() == want_s.view(np.uint32).tobytes(), f"{name} scales"


@pytest.mark.parametrize("paged", [False, True])
def test_int8_append_is_bit_exact(paged):
    """Quantising append: the oracle's codes and scales, untouched slots kept."""
    _append_case(paged)


@pytest.mark.parametrize("H,K", [(32, 8), (64, 8), (16, 16), (8, 8), (64, 1), (24, 8)])
def test_int8_decode_matches_oracle(H, K):
    _decode_case(LLAMA3.replace(B=5, H=H, K=K, ctx=("uniform", 1, 900)), f"H={H} K={K}", codec="int8")


@pytest.mark.parametrize("window", [1, 33, 500])
def test_int8_decode_window(window):
    _decode_case(LLAMA3.replace(B=4, ctx=("uniform", 100, 1500)), f"window {window}", window=window, codec="int8")


@pytest.mark.parametrize("block_size", [16, 64])
def test_int8_decode_paged(block_size):
    wl = W.WORKLOADS["paged_long_decode"].replace(B=4, ctx=("loguniform", 20, 2500), block_size=block_size)
    _decode_case(wl, f"paged bs={block_size}", codec="int8")


def test_int8_decode_full_size_sampled():
    _decode_case(LLAMA3, "llama3_8b_decode shape", seqs=[0, 13, 31], codec="int8")


def test_int8_decode_step_quantises_the_new_token():
    """gqa_decode_step on an INT8 cache: the new token is quantised as the
    append does it and attended to."""
    wl = LLAMA3.replace(B=4, ctx=("uniform", 1, 600))
    inp = W.make_decode(wl, fill="zero")
    kc, ks, vc, vs = quantized_inputs(inp, "int8")
    kn, vn = inp.new_token_rows()
    kc0, ks0, vc0, vs0 = kc.copy(), ks.copy(), vc.copy(), vs.copy()
    for b in range(wl.B):
        t = int(inp.ctx[b]) - 1
        for c, s in ((kc0, ks0), (vc0, vs0)):
            c[b, :, t] = 0x80
            s[b, :, t] = np.nan
    cache = _f8_cache(kc0, ks0, vc0, vs0, None, "int8")
    say("int8 decode step")
    out = binding.gqa_decode_step(to_dev(inp.q), to_dev(kn), to_dev(vn), cache, to_dev(inp.ctx),
                                  int(inp.ctx.max()), scale=wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(f8_host(cache.k), kc) and np.array_equal(f8_host(cache.v), vc)
    assert np.array_equal(cache.k_scale.cpu().numpy(), ks, equal_nan=True)
    assert np.array_equal(cache.v_scale.cpu().numpy(), vs, equal_nan=True)
    rows, want = oracle_rows_f8(inp, kc, ks, vc, vs, range(wl.B), codec="int8")
    got = as_f64(from_dev(out)[rows[:, 0], rows[:, 1], rows[:, 2]], "bf16")
    check_close(got, want, BF16_TOL, "int8 decode step")


@pytest.mark.parametrize("s_new,H,K", [(4, 32, 8), (8, 64, 8)])
def test_int8_decode_multi_matches_causal_oracle(s_new, H, K):
    """Several newest positions per sequence on an INT8 cache: row i at
    ctx - s + i attends causally to the dequantised keys."""
    wl = LLAMA3.replace(B=4, H=H, K=K, ctx=("uniform", 16, 900))
    inp = W.make_decode(wl, fill="zero")
    kc, ks, vc, vs = quantized_inputs(inp, "int8")
    cache = _f8_cache(kc, ks, vc, vs, inp.block_table, "int8")
    rng = np.random.default_rng(wl.seed + 5)
    q = W.f32_to_bf16_bits(rng.standard_normal((wl.B, s_new, wl.H, wl.d)).astype(np.float32))
    say("int8 decode multi", f"s={s_new} H={H} K={K}")
    out = binding.gqa_decode_multi(to_dev(q), cache, to_dev(inp.ctx), int(inp.ctx.max()), scale=wl.scale)
    torch.cuda.synchronize()
    o = from_dev(out)
    kd, vd = dequant(kc, ks, "int8"), dequant(vc, vs, "int8")
    got, want = [], []
    for b in range(wl.B):
        n = int(inp.ctx[b])
        rows = np.array([[0, i, h] for i in range(s_new) for h in range(wl.H)], dtype=np.int32)
        want.append(oracle.attention_rows(as_f64(q[b:b + 1], "bf16"), kd[b:b + 1, :, :n], vd[b:b + 1, :, :n],
                                          [n - s_new], [n], True, wl.scale, rows))
        got.append(as_f64(o[b][rows[:, 1], rows[:, 2]], "bf16"))
    check_close(np.concatenate(got), np.concatenate(want), BF16_TOL, f"int8 decode multi s={s_new}")


# ---------------------------------------------------------------------------
# exact coverage of the paged INT8 decode: V rows are integers times a
# power-of-two step with one element at 127 steps, so their scale is that
# step and the round trip is exact
# ---------------------------------------------------------------------------

def _paged_i8_structured(ctx, starts, width, spike, seed, H=64, K=8):
    """Group g of sequence b puts all its weight on the cached keys
    [starts[b][g], + width): K rows there are 2.5 u (u the group's query row),
    zero elsewhere."""
    wl = W.WORKLOADS["paged_long_decode"].replace(B=len(ctx), H=H, K=K)
    rng = np.random.default_rng(seed)
    inp = W.make_decode(wl, fill="zero", ctx_override=ctx)
    bs, d = wl.block_size, wl.d
    u = rng.choice([-1.0, 1.0], size=(wl.B, wl.K, d)).astype(np.float32)
    for b in range(wl.B):
        n = int(ctx[b])
        t = np.arange(n)
        blk, slot = inp.block_table[b, t // bs].astype(np.int64), t % bs
        for g in range(wl.K):
            inp.q[b, 0, g * wl.G:(g + 1) * wl.G] = BF16(u[b, g])
            lo = int(starts[b][g])
            inside = (t >= lo) & (t < lo + width)
            inp.k[blk, g, slot] = BF16(np.where(inside[:, None], 2.5 * u[b, g][None, :], 0.0))
            if spike:
                # no zero code: the other keys' tiny weights (~e^-40 each) then
                # vanish in the bf16 output beside every element of the spike row
                m = rng.integers(1, 128, size=(n, d)).astype(np.float64) * rng.choice([-1.0, 1.0], size=(n, d))
                m[:, 0] = 127.0 * rng.choice([-1.0, 1.0], size=n)
                inp.v[blk, g, slot] = BF16(m * np.exp2((t % 5) - 9.0)[:, None])
            else:
                rows = np.zeros((n, d), np.float32)
                rows[t, t % d] = 127.0 / 64.0   # scale 1/64, code 127
                inp.v[blk, g, slot] = BF16(rows)
    kc, ks, vc, vs = quantized_inputs(inp, "int8")
    return wl, inp, kc, ks, vc, vs


def _run_i8(wl, inp, kc, ks, vc, vs, what):
    cache = _f8_cache(kc, ks, vc, vs, inp.block_table, "int8")
    say("int8 paged exact", what)
    out = binding.gqa_decode(to_dev(inp.q), cache, to_dev(inp.ctx), int(inp.ctx.max()), scale=wl.scale)
    torch.cuda.synchronize()
    return from_dev(out)


def test_int8_paged_window_coverage_exact():
    ctx = np.array([128, 1000, 3001, 4096], np.int32)
    starts = []
    for n in ctx:
        n = int(n)
        cand = [0, n - 128, 16 * ((n - 128) // 32), max(0, n - 135), (n - 128) // 3, 1 % max(1, n - 127), 17, 31]
        starts.append([max(0, min(n - 128, c)) for c in cand])
    wl, inp, kc, ks, vc, vs = _paged_i8_structured(ctx, starts, 128, False, 43)
    assert (vs[inp.block_table[0, 0], 0, :1] == np.float32(1.0 / 64.0)).all()
    out = as_f64(_run_i8(wl, inp, kc, ks, vc, vs, "window"), "bf16")
    assert np.array_equal(out, np.full(out.shape, 127.0 / 64.0 / 128.0)), starts


def test_int8_paged_spikes_exact():
    """One cached key per (sequence, group): the first or last slot of a block or
    the last valid slot.  Every head of the group returns the oracle's
    dequantised V row of that key bit for bit."""
    ctx = np.array([520, 1601, 33, 4000], np.int32)
    starts = []
    for n in ctx:
        n = int(n)
        cand = [0, 15, 16, 31, 32, n - 1, n - 16, (n // 2) // 16 * 16 - 1]
        starts.append([max(0, min(n - 1, c)) for c in cand])
    wl, inp, kc, ks, vc, vs = _paged_i8_structured(ctx, starts, 1, True, 44)
    vd = dequant(vc, vs, "int8")
    out = as_f64(_run_i8(wl, inp, kc, ks, vc, vs, "spikes"), "bf16")
    for b in range(wl.B):
        for g in range(wl.K):
            t = starts[b][g]
            blk, slot = int(inp.block_table[b, t // 16]), t % 16
            want = vd[blk, g, slot]
            assert np.array_equal(want, as_f64(inp.v[blk, g, slot], "bf16"))   # the round trip is exact
            for r in range(wl.G):
                assert np.array_equal(out[b, 0, g * wl.G + r], want), (b, g, t)


# ---------------------------------------------------------------------------
# prefill over an INT8 cache (inference-optimisation page §11.7 with §15.5.1)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("H,K", [(32, 8), (64, 8), (8, 8), (64, 1)])
def test_int8_prefill_matches_oracle(H, K):
    _check_fp8_prefill(f"int8 prefill H={H} K={K}", B=2, H=H, K=K, s=150, start=0, seed=H + K, codec="int8")


@pytest.mark.parametrize("paged,bs", [(False, 16), (True, 16), (True, 4), (True, 64)])
def test_int8_prefill_after_a_quantised_prefix(paged, bs):
    _check_fp8_prefill(f"int8 chunked prefill paged={paged} bs={bs}", B=3, H=32, K=8, s=70, start=[200, 63, 1],
                       paged=paged, bs=bs, seed=bs, codec="int8")


@pytest.mark.parametrize("window,causal", [(40, True), (0, False)])
def test_int8_prefill_window_and_full(window, causal):
    _check_fp8_prefill(f"int8 prefill window={window} causal={causal}", B=2, H=32, K=8, s=100, start=[90, 17],
                       window=window, causal=causal, seed=7, codec="int8")


def test_int8_chunked_prefill_full_size_sampled():
    """The bench's chunked shape on an INT8 cache: 512 new tokens after a
    3584-token quantised prefix in shuffled 16-token blocks; 300 sampled rows."""
    rng = np.random.default_rng(10)
    B, H, s = 4, 32, 512
    rows = np.stack([rng.integers(0, B, 300), rng.integers(0, s, 300), rng.integers(0, H, 300)], axis=1).astype(np.int32)
    rows[:4] = [[0, 0, 0], [3, s - 1, H - 1], [1, 255, 17], [2, 511, 3]]
    _check_fp8_prefill("int8 chunked prefill, full size", B=B, H=H, K=8, s=s, start=3584, paged=True, rows=rows,
                       seed=4, codec="int8")
