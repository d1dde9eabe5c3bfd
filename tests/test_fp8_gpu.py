"""FP8 (E4M3) KV cache with one fp32 scale per cached row (inference-
optimisation page §15.5-§15.5.1: per-token / per-head scales, FP8 E4M3),
through the C ABI, against the oracle.

* The quantising append must give the oracle's codes and scales bit for bit
  (both decide in fp32: scale = amax / 448, code = E4M3(x / scale)).
* Decode on a quantised cache must match the fp64 oracle attention over the
  dequantised values (scale * E4M3(code)) within the bf16 tolerance.
Unused cache slots hold the NaN code and NaN scales, so a read of one shows."""
import numpy as np
import pytest
import torch

import oracle
from grouped_query_attention_gqa_amd import binding
from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import BF16_TOL, as_f64, check_close, from_dev, say, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

NAN_CODE = 0x7F
# The helpers below take codec="fp8" (E4M3) or "int8" (tests/test_int8_gpu.py):
# the quantiser and decoder of the oracle, the torch dtype of the codes and
# the code that fills unused slots (the E4M3 NaN code; -128, a code the INT8
# quantiser never writes).
QUANT = {"fp8": (oracle.quantize_e4m3_rows, oracle.dequantize_e4m3_rows, torch.float8_e4m3fn, NAN_CODE),
         "int8": (oracle.quantize_i8_rows, oracle.dequantize_i8_rows, torch.int8, 0x80)}


def f8_dev(codes: np.ndarray, codec: str = "fp8") -> torch.Tensor:
    """Codes (uint8 bytes or int8) on the device, as the codec's torch dtype."""
    raw = np.ascontiguousarray(codes).view(np.uint8)
    return torch.from_numpy(raw).to("cuda").view(QUANT[codec][2])


def f8_host(t: torch.Tensor) -> np.ndarray:
    """The code bytes of a device tensor (uint8)."""
    return t.detach().view(torch.uint8).cpu().numpy()


def _used_slots(inp: W.DecodeInputs) -> np.ndarray:
    """Boolean mask over the cache rows [.., .., slots] that hold a visible token."""
    wl = inp.wl
    if inp.block_table is None:
        used = np.zeros(inp.k.shape[:3], dtype=bool)
        for b in range(wl.B):
            used[b, :, :int(inp.ctx[b])] = True
        return used
    used = np.zeros(inp.k.shape[:3], dtype=bool)
    bs = wl.block_size
    for b in range(wl.B):
        for t in range(int(inp.ctx[b])):
            used[int(inp.block_table[b, t // bs]), :, t % bs] = True
    return used


def quantized_inputs(inp: W.DecodeInputs, codec: str = "fp8"):
    """The oracle's codes (as uint8 bytes) and scales of the (zero-filled) bf16
    cache, with every unused slot set to the fill code and a NaN scale."""
    quant = QUANT[codec][0]
    kc, ks = quant(inp.k)
    vc, vs = quant(inp.v)
    kc, vc = kc.view(np.uint8), vc.view(np.uint8)
    used = _used_slots(inp)
    for c, s in ((kc, ks), (vc, vs)):
        c[~used] = QUANT[codec][3]
        s[~used] = np.nan
    return kc, ks, vc, vs


def dequant(codes, scales, codec: str = "fp8"):
    """The oracle's values of code bytes and scales."""
    return QUANT[codec][1](codes.view(np.int8) if codec == "int8" else codes, scales)


def oracle_rows_f8(inp, kc, ks, vc, vs, seqs, window=0, codec: str = "fp8"):
    """fp64 oracle attention over the dequantised cache for the listed sequences."""
    wl = inp.wl
    kd = dequant(kc, ks, codec)
    vd = dequant(vc, vs, codec)
    rows_all, outs = [], []
    for b in seqs:
        n = int(inp.ctx[b])
        if inp.block_table is None:
            kb, vb = kd[b:b + 1, :, :n], vd[b:b + 1, :, :n]
        else:
            bs = wl.block_size
            idx = [(int(inp.block_table[b, t // bs]), t % bs) for t in range(n)]
            kb = np.stack([kd[blk, :, s] for blk, s in idx], axis=1)[None]
            vb = np.stack([vd[blk, :, s] for blk, s in idx], axis=1)[None]
        rows = np.array([[0, 0, h] for h in range(wl.H)], dtype=np.int32)
        o = oracle.attention_rows(as_f64(inp.q[b:b + 1], "bf16"), kb, vb, [n - 1], [n], False, wl.scale, rows,
                                  window)
        rows[:, 0] = b
        rows_all.append(rows)
        outs.append(o)
    return np.concatenate(rows_all), np.concatenate(outs)


def _f8_cache(kc, ks, vc, vs, table, codec: str = "fp8"):
    return binding.KVCache(f8_dev(kc, codec), f8_dev(vc, codec), None if table is None else to_dev(table),
                           k_scale=to_dev(ks), v_scale=to_dev(vs))


def _decode_case(wl, what, window=0, seqs=None, codec: str = "fp8"):
    inp = W.make_decode(wl, fill="zero")
    kc, ks, vc, vs = quantized_inputs(inp, codec)
    cache = _f8_cache(kc, ks, vc, vs, inp.block_table, codec)
    seqs = list(range(wl.B)) if seqs is None else seqs
    say(f"{codec} decode", what, f"window={window}")
    out = binding.gqa_decode(to_dev(inp.q), cache, to_dev(inp.ctx), int(inp.ctx.max()), scale=wl.scale,
                             window=window)
    torch.cuda.synchronize()
    o = from_dev(out)
    rows, want = oracle_rows_f8(inp, kc, ks, vc, vs, seqs, window, codec)
    got = as_f64(o[rows[:, 0], rows[:, 1], rows[:, 2]], "bf16")
    check_close(got, want, BF16_TOL, f"{codec} decode {what}")


LLAMA3 = W.WORKLOADS["llama3_8b_decode"]


def test_fp8_append_is_bit_exact():
    """Quantising append: the oracle's codes and scales, untouched slots kept."""
    rng = np.random.default_rng(11)
    B, s_new, K, d, S = 3, 5, 8, 128, 40
    kn = W.f32_to_bf16_bits(rng.standard_normal((B, s_new, K, d)).astype(np.float32)
                     * rng.lognormal(0, 2, (B, s_new, K, 1)).astype(np.float32))
    vn = W.f32_to_bf16_bits(rng.standard_normal((B, s_new, K, d)).astype(np.float32))
    kn[0, 0, 0] = 0                                   # an all-zero row
    kn[1, 2, 3] = W.f32_to_bf16_bits(np.float32([1e-3] * d))
    kn[1, 2, 3, 7] = W.f32_to_bf16_bits(np.float32([-3.0e4]))[0]   # one large negative value
    start = np.array([0, 17, 37], dtype=np.int32)      # the last one runs past S_max: those rows are skipped
    codes0 = np.full((B, K, S, d), 0xAB, dtype=np.uint8)
    scales0 = np.full((B, K, S), np.nan, dtype=np.float32)
    kcache, vcache = f8_dev(codes0), f8_dev(codes0)
    ksc, vsc = to_dev(scales0), to_dev(scales0)
    cache = binding.KVCache(kcache, vcache, None, k_scale=ksc, v_scale=vsc)
    say("fp8 append")
    binding.gqa_kv_append(cache, to_dev(kn), to_dev(vn), to_dev(start))
    torch.cuda.synchronize()
    for name, new, codes_d, sc_d in (("k", kn, kcache, ksc), ("v", vn, vcache, vsc)):
        want_c, want_s = codes0.copy(), scales0.copy()
        qc, qs = oracle.quantize_e4m3_rows(new)        # [B, s_new, K, d], [B, s_new, K]
        for b in range(B):
            for t in range(s_new):
                pos = start[b] + t
                if pos < S:
                    want_c[b, :, pos] = qc[b, t]
                    want_s[b, :, pos] = qs[b, t]
        got_c, got_s = f8_host(codes_d), sc_d.cpu().numpy()
        assert np.array_equal(got_c, want_c), f"{name} codes differ"
        assert got_s.view(np.uint32).tobytes() == want_s.view(np.uint32).tobytes(), f"{name} scales differ"


def test_fp8_append_paged_is_bit_exact():
    rng = np.random.default_rng(12)
    B, s_new, K, d, bs = 2, 20, 8, 128, 16
    kn = W.f32_to_bf16_bits(rng.standard_normal((B, s_new, K, d)).astype(np.float32))
    vn = W.f32_to_bf16_bits(rng.standard_normal((B, s_new, K, d)).astype(np.float32) * 7)
    table = np.array([[3, 0, 5], [1, 4, 2]], dtype=np.int32)
    start = np.array([9, 0], dtype=np.int32)
    N = 6
    codes0 = np.full((N, K, bs, d), 0xAB, dtype=np.uint8)
    scales0 = np.full((N, K, bs), np.nan, dtype=np.float32)
    kp, vp, ksc, vsc = f8_dev(codes0), f8_dev(codes0), to_dev(scales0), to_dev(scales0)
    cache = binding.KVCache(kp, vp, to_dev(table), k_scale=ksc, v_scale=vsc)
    say("fp8 append paged")
    binding.gqa_kv_append(cache, to_dev(kn), to_dev(vn), to_dev(start))
    torch.cuda.synchronize()
    for name, new, codes_d, sc_d in (("k", kn, kp, ksc), ("v", vn, vp, vsc)):
        want_c, want_s = codes0.copy(), scales0.copy()
        qc, qs = oracle.quantize_e4m3_rows(new)
        for b in range(B):
            for t in range(s_new):
                pos = start[b] + t
                blk = table[b, pos // bs]
                want_c[blk, :, pos % bs] = qc[b, t]
                want_s[blk, :, pos % bs] = qs[b, t]
        assert np.array_equal(f8_host(codes_d), want_c), f"{name} codes differ"
        assert sc_d.cpu().numpy().view(np.uint32).tobytes() == want_s.view(np.uint32).tobytes(), f"{name} scales"


@pytest.mark.parametrize("H,K", [(32, 8), (64, 8), (16, 16), (16, 8), (8, 8), (64, 4), (64, 1), (24, 8)])
def test_fp8_decode_matches_oracle(H, K):
    _decode_case(LLAMA3.replace(B=5, H=H, K=K, ctx=("uniform", 1, 900)), f"H={H} K={K}")


@pytest.mark.parametrize("window", [1, 33, 500])
def test_fp8_decode_window(window):
    _decode_case(LLAMA3.replace(B=4, ctx=("uniform", 100, 1500)), f"window {window}", window=window)


@pytest.mark.parametrize("block_size", [16, 64])
def test_fp8_decode_paged(block_size):
    wl = W.WORKLOADS["paged_long_decode"].replace(B=4, ctx=("loguniform", 20, 2500), block_size=block_size)
    _decode_case(wl, f"paged bs={block_size}")


def test_fp8_decode_full_size_sampled():
    _decode_case(LLAMA3, "llama3_8b_decode shape", seqs=[0, 13, 31])


def test_fp8_decode_step_quantises_the_new_token():
    """gqa_decode_step on an FP8 cache: the new token is quantised as the append
    does it and attended to."""
    wl = LLAMA3.replace(B=4, ctx=("uniform", 1, 600))
    inp = W.make_decode(wl, fill="zero")
    kc, ks, vc, vs = quantized_inputs(inp)
    kn, vn = inp.new_token_rows()
    # the slot being filled starts as NaN code / NaN scale on the device
    kc0, ks0, vc0, vs0 = kc.copy(), ks.copy(), vc.copy(), vs.copy()
    for b in range(wl.B):
        t = int(inp.ctx[b]) - 1
        for c, s in ((kc0, ks0), (vc0, vs0)):
            c[b, :, t] = NAN_CODE
            s[b, :, t] = np.nan
    cache = _f8_cache(kc0, ks0, vc0, vs0, None)
    say("fp8 decode step")
    out = binding.gqa_decode_step(to_dev(inp.q), to_dev(kn), to_dev(vn), cache, to_dev(inp.ctx),
                                  int(inp.ctx.max()), scale=wl.scale)
    torch.cuda.synchronize()
    assert np.array_equal(f8_host(cache.k), kc) and np.array_equal(f8_host(cache.v), vc)
    assert np.array_equal(cache.k_scale.cpu().numpy(), ks, equal_nan=True)
    rows, want = oracle_rows_f8(inp, kc, ks, vc, vs, range(wl.B))
    got = as_f64(from_dev(out)[rows[:, 0], rows[:, 1], rows[:, 2]], "bf16")
    check_close(got, want, BF16_TOL, "fp8 decode step")


def test_fp8_single_key_returns_the_dequantised_value():
    """ctx = 1: the output is the one dequantised V row (up to the bf16 rounding
    of the scale-carrying probability and of the output)."""
    wl = LLAMA3.replace(B=2, ctx=("fixed", 1))
    _decode_case(wl, "ctx 1")


@pytest.mark.parametrize("s_new,H,K", [(4, 32, 8), (2, 64, 8), (8, 64, 8)])
def test_fp8_decode_multi_matches_causal_oracle(s_new, H, K):
    """Several newest positions per sequence on an FP8 cache: row i at
    ctx - s + i attends causally to the dequantised keys."""
    wl = LLAMA3.replace(B=4, H=H, K=K, ctx=("uniform", 16, 900))
    inp = W.make_decode(wl, fill="zero")
    kc, ks, vc, vs = quantized_inputs(inp)
    cache = _f8_cache(kc, ks, vc, vs, inp.block_table)
    rng = np.random.default_rng(wl.seed + 5)
    q = W.f32_to_bf16_bits(rng.standard_normal((wl.B, s_new, wl.H, wl.d)).astype(np.float32))
    say("fp8 decode multi", f"s={s_new} H={H} K={K}")
    out = binding.gqa_decode_multi(to_dev(q), cache, to_dev(inp.ctx), int(inp.ctx.max()), scale=wl.scale)
    torch.cuda.synchronize()
    o = from_dev(out)
    kd = oracle.dequantize_e4m3_rows(kc, ks)
    vd = oracle.dequantize_e4m3_rows(vc, vs)
    got, want = [], []
    for b in range(wl.B):
        n = int(inp.ctx[b])
        rows = np.array([[0, i, h] for i in range(s_new) for h in range(wl.H)], dtype=np.int32)
        want.append(oracle.attention_rows(as_f64(q[b:b + 1], "bf16"), kd[b:b + 1, :, :n], vd[b:b + 1, :, :n],
                                          [n - s_new], [n], True, wl.scale, rows))
        got.append(as_f64(o[b][rows[:, 1], rows[:, 2]], "bf16"))
    check_close(np.concatenate(got), np.concatenate(want), BF16_TOL, f"fp8 decode multi s={s_new}")


# ---------------------------------------------------------------------------
# exact coverage of the paged FP8 decode: the block table walk and the scales
# it loads beside the codes (a wrong block, slot or scale changes an output
# bit).  The values are chosen so that the FP8 round trip is exact: every V
# row's scale is a power of two (amax = 1.75 * 2^e, so scale = 2^(e-8)) and
# its values have at most three mantissa bits.
# ---------------------------------------------------------------------------

BF16 = lambda x: W.f32_to_bf16_bits(np.asarray(x, np.float32))


def _paged_f8_structured(ctx, starts, width, spike, seed, H=64, K=8):
    """Paged FP8 inputs whose group g of sequence b puts all its weight on the
    cached keys [starts[b][g], + width): K rows there are 2.5 u (u the group's
    query row), zero elsewhere."""
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
                sign = rng.choice([-1.0, 1.0], size=(n, d))
                mant = 1.0 + ((t[:, None] + np.arange(d)[None, :]) % 7) / 8.0     # 1 .. 1.75: amax 1.75
                inp.v[blk, g, slot] = BF16(sign * mant * np.exp2((t % 5) - 2.0)[:, None])
            else:
                rows = np.zeros((n, d), np.float32)
                rows[t, t % d] = 1.75
                inp.v[blk, g, slot] = BF16(rows)
    kc, ks, vc, vs = quantized_inputs(inp)
    return wl, inp, kc, ks, vc, vs


def _run_f8(wl, inp, kc, ks, vc, vs, what, window=0):
    cache = _f8_cache(kc, ks, vc, vs, inp.block_table)
    say("fp8 paged exact", what)
    out = binding.gqa_decode(to_dev(inp.q), cache, to_dev(inp.ctx), int(inp.ctx.max()), scale=wl.scale,
                             window=window)
    torch.cuda.synchronize()
    return from_dev(out)


def test_fp8_paged_window_coverage_exact():
    ctx = np.array([128, 1000, 3001, 4096], np.int32)
    starts = []
    for n in ctx:
        n = int(n)
        cand = [0, n - 128, 16 * ((n - 128) // 32), max(0, n - 135), (n - 128) // 3, 1 % max(1, n - 127), 17, 31]
        starts.append([max(0, min(n - 128, c)) for c in cand])
    wl, inp, kc, ks, vc, vs = _paged_f8_structured(ctx, starts, 128, False, 41)
    # one-hot rows of 1.75: scale 2^-8, code 448, value 1.75 exactly
    assert (vs[inp.block_table[0, 0], 0, :1] == np.float32(2.0 ** -8)).all()
    out = as_f64(_run_f8(wl, inp, kc, ks, vc, vs, "window"), "bf16")
    assert np.array_equal(out, np.full(out.shape, 1.75 / 128.0)), starts


def test_fp8_paged_spikes_exact():
    """One cached key per (sequence, group): the first or last slot of a block or
    the last valid slot.  Every head of the group returns the oracle's
    dequantised V row of that key bit for bit."""
    ctx = np.array([520, 1601, 33, 4000], np.int32)
    starts = []
    for n in ctx:
        n = int(n)
        cand = [0, 15, 16, 31, 32, n - 1, n - 16, (n // 2) // 16 * 16 - 1]
        starts.append([max(0, min(n - 1, c)) for c in cand])
    wl, inp, kc, ks, vc, vs = _paged_f8_structured(ctx, starts, 1, True, 42)
    vd = oracle.dequantize_e4m3_rows(vc, vs)
    out = as_f64(_run_f8(wl, inp, kc, ks, vc, vs, "spikes"), "bf16")
    for b in range(wl.B):
        for g in range(wl.K):
            t = starts[b][g]
            blk, slot = int(inp.block_table[b, t // 16]), t % 16
            want = vd[blk, g, slot]
            # the round trip through E4M3 is exact for these rows
            assert np.array_equal(want, as_f64(inp.v[blk, g, slot], "bf16"))
            for r in range(wl.G):
                assert np.array_equal(out[b, 0, g * wl.G + r], want), (b, g, t)


# ---------------------------------------------------------------------------
# prefill over an FP8 cache (inference-optimisation page §11.7 with §15.5.1):
# the new rows are quantised into the cache by the call, and every row, old
# and new, is read as scale * E4M3(code); the oracle is the plain attention
# over those values (oracle.prefill_fp8_rows).
# ---------------------------------------------------------------------------

def _fp8_prefill_run(B, H, K, s, start, *, paged=False, bs=16, causal=True, window=0, seed=0, rows=None,
                     inputs=None, codec="fp8"):
    """Runs gqa_prefill on an FP8 cache holding start[b] quantised prefix tokens
    of sequence b; returns (out [B,s,H,d] bf16 bits, expected rows, rows).
    inputs = (q, k_new, v_new, k_prefix, v_prefix) as bf16 bits, else random.
    Unused cache slots hold the NaN code and NaN scales; the cache after the
    call must be the oracle's quantising append of the new rows, bit for bit."""
    d = 128
    rng = np.random.default_rng(seed)
    starts = np.full(B, start, np.int32) if np.isscalar(start) else np.asarray(start, np.int32)
    S = int(starts.max()) + s
    if inputs is None:
        bits = lambda *shape, f=1.0: W.f32_to_bf16_bits((rng.standard_normal(shape) * 0.5 * f).astype(np.float32))
        q, kn, vn = bits(B, s, H, d), bits(B, s, K, d), bits(B, s, K, d)
        kp = bits(B, S, K, d, f=rng.lognormal(0, 1, (B, S, K, 1)))
        vp = bits(B, S, K, d)
    else:
        q, kn, vn, kp, vp = inputs
    table = None
    if paged:
        table, n_pool = W.deal_blocks(rng, starts + s, bs, slack_blocks=2)
        shape = (n_pool, K, bs, d)
    else:
        shape = (B, K, S, d)
    cdt = np.int8 if codec == "int8" else np.uint8
    codes = {n: np.full(shape, QUANT[codec][3], np.uint8).view(cdt) for n in "kv"}
    scales = {n: np.full(shape[:-1], np.nan, np.float32) for n in "kv"}
    # the prefix: positions t < starts[b] of sequence b, quantised by the oracle
    for n, pre in (("k", kp), ("v", vp)):
        for b in range(B):
            if starts[b] == 0:
                continue
            rows_b = np.ascontiguousarray(pre[b:b + 1, :starts[b]])
            if table is None:
                c, sc = oracle.fp8_cache_after_append(codes[n][b:b + 1], scales[n][b:b + 1], rows_b, [0],
                                                      codec=codec)
                codes[n][b], scales[n][b] = c[0], sc[0]
            else:
                codes[n], scales[n] = oracle.fp8_cache_after_append(codes[n], scales[n], rows_b, [0], table[b:b + 1],
                                                                    codec=codec)
    cache = _f8_cache(codes["k"], scales["k"], codes["v"], scales["v"], table, codec)
    say(f"{codec} prefill", f"B={B} H={H} K={K} s={s} start={list(starts)} paged={paged} bs={bs} window={window}")
    out = binding.gqa_prefill(to_dev(q), to_dev(kn), to_dev(vn), cache, to_dev(starts), causal=causal,
                              scale=1.0 / np.sqrt(d), window=window)
    torch.cuda.synchronize()
    after = {}
    for n, new in (("k", kn), ("v", vn)):
        want_c, want_s = oracle.fp8_cache_after_append(codes[n], scales[n], new, starts, table, codec=codec)
        got_c = f8_host(getattr(cache, n)).view(cdt)
        got_s = getattr(cache, n + "_scale").cpu().numpy()
        assert np.array_equal(got_c, want_c), f"{n} codes after the prefill"
        assert got_s.view(np.uint32).tobytes() == want_s.view(np.uint32).tobytes(), f"{n} scales after the prefill"
        after[n] = (want_c, want_s)
    if rows is None:
        rows = np.array([[b, i, h] for b in range(B) for i in range(s) for h in range(H)], np.int32)
    want = oracle.prefill_fp8_rows(as_f64(q, "bf16"), after["k"][0], after["k"][1], after["v"][0], after["v"][1],
                                   starts, s, causal, 1.0 / np.sqrt(d), rows, window, table, codec=codec)
    return from_dev(out), want, rows, after, table


def _check_fp8_prefill(what, **kw):
    out, want, rows, _, _ = _fp8_prefill_run(**kw)
    got = as_f64(out[rows[:, 0], rows[:, 1], rows[:, 2]], "bf16")
    check_close(got, want, BF16_TOL, what)


@pytest.mark.parametrize("H,K", [(32, 8), (64, 8), (8, 8), (64, 1), (24, 8)])
def test_fp8_prefill_matches_oracle(H, K):
    _check_fp8_prefill(f"fp8 prefill H={H} K={K}", B=2, H=H, K=K, s=150, start=0, seed=H + K)


@pytest.mark.parametrize("paged,bs", [(False, 16), (True, 16), (True, 4), (True, 64)])
def test_fp8_prefill_after_a_quantised_prefix(paged, bs):
    _check_fp8_prefill(f"fp8 chunked prefill paged={paged} bs={bs}", B=3, H=32, K=8, s=70, start=[200, 63, 1],
                       paged=paged, bs=bs, seed=bs)


@pytest.mark.parametrize("window,causal", [(40, True), (1, True), (0, False)])
def test_fp8_prefill_window_and_full(window, causal):
    _check_fp8_prefill(f"fp8 prefill window={window} causal={causal}", B=2, H=32, K=8, s=100, start=[90, 17],
                       window=window, causal=causal, seed=7)


def test_fp8_chunked_prefill_full_size_sampled():
    """The bench's chunked shape on an FP8 cache: 512 new tokens after a
    3584-token quantised prefix in shuffled 16-token blocks; 300 sampled rows."""
    rng = np.random.default_rng(9)
    B, H, s = 4, 32, 512
    rows = np.stack([rng.integers(0, B, 300), rng.integers(0, s, 300), rng.integers(0, H, 300)], axis=1).astype(np.int32)
    rows[:4] = [[0, 0, 0], [3, s - 1, H - 1], [1, 255, 17], [2, 511, 3]]
    _check_fp8_prefill("fp8 chunked prefill, full size", B=B, H=H, K=8, s=s, start=3584, paged=True, rows=rows,
                       seed=3)


def test_fp8_prefill_spikes_over_the_prefix_exact():
    """All weight on one cached key per (sequence, group), the first or last slot
    of a block or the prefix's last slot, whose V row has a power-of-two scale:
    every new row of the group returns that dequantised row bit for bit."""
    B, H, K, d, s, start = 2, 32, 8, 128, 64, 1000
    G = H // K
    rng = np.random.default_rng(61)
    u = rng.choice([-1.0, 1.0], size=(B, K, d)).astype(np.float32)
    kp = np.zeros((B, start, K, d), np.float32)
    t = np.arange(start)
    mant = 1.0 + ((t[:, None] + np.arange(d)[None, :]) % 7) / 8.0          # 1 .. 1.75: amax 1.75
    vp = (rng.choice([-1.0, 1.0], size=(B, start, K, d)) * mant[None, :, None, :] *
          np.exp2((t % 5) - 2.0)[None, :, None, None]).astype(np.float32)
    spikes = [[0, 15, 16, 999, 511, 512, 31, 640], [1, 14, 999, 998, 32, 47, 48, 100]]
    for b in range(B):
        for g in range(K):
            kp[b, spikes[b][g], g] = 2.5 * u[b, g]
    q = np.zeros((B, s, H, d), np.float32)
    for g in range(K):
        q[:, :, g * G:(g + 1) * G] = u[:, g][:, None, None, :]
    kn = np.zeros((B, s, K, d), np.float32)
    vn = rng.standard_normal((B, s, K, d)).astype(np.float32)
    bits = W.f32_to_bf16_bits
    out, want, rows, after, table = _fp8_prefill_run(B=B, H=H, K=K, s=s, start=start, paged=True, seed=62,
                                                     inputs=(bits(q), bits(kn), bits(vn), bits(kp), bits(vp)))
    vd = oracle.dequantize_e4m3_rows(*after["v"])
    got = as_f64(out, "bf16")
    for b in range(B):
        for g in range(K):
            tt = spikes[b][g]
            want_row = vd[int(table[b, tt // 16]), g, tt % 16]
            assert np.array_equal(want_row, vp[b, tt, g].astype(np.float64))   # the round trip is exact here
            assert np.array_equal(got[b, :, g * G:(g + 1) * G], np.broadcast_to(want_row, (s, G, d))), (b, g, tt)
    check_close(got[rows[:, 0], rows[:, 1], rows[:, 2]], want, BF16_TOL, "fp8 spikes against the oracle")
