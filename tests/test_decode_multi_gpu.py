"""Decode on the matrix cores: large groups (G = 16 .. 64, the multi-query end,
through gqa_decode) and several newest positions per sequence at once
(gqa_decode_multi), through the C ABI, against the oracle.

Row i of a block of s positions sits at ctx - s + i and attends causally
(the concept page's rule that a token sees itself and every earlier token);
the oracle computes exactly that as a prefill of the s rows after ctx - s
cached tokens.  Unused cache slots hold NaN."""
import numpy as np
import pytest
import torch

import oracle
from grouped_query_attention_gqa_amd import binding
from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import (BF16_TOL, DecodeRun, as_f64, check_close, from_dev, gpu_rows, oracle_decode_rows, say,
                        to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

LLAMA70 = W.WORKLOADS["llama2_70b_decode"]


# G = 64 and 40 run as two items of G / 2 heads, G = 33 on the 64-row kernel
@pytest.mark.parametrize("H,K", [(64, 4), (64, 2), (64, 1), (48, 3), (32, 1), (33, 1), (40, 1)])
def test_large_group_decode(H, K):
    wl = LLAMA70.replace(B=5, H=H, K=K, ctx=("uniform", 1, 1500))
    inp = W.make_decode(wl)
    say("mfma decode", f"H={H} K={K}")
    out = from_dev(DecodeRun(inp).run())
    rows, want = oracle_decode_rows(inp)
    check_close(gpu_rows(out, rows, "bf16"), want, BF16_TOL, f"G={H // K} decode")


@pytest.mark.parametrize("window", [1, 40, 700])
def test_large_group_decode_window(window):
    wl = LLAMA70.replace(B=4, H=64, K=2, ctx=("uniform", 50, 2000))
    inp = W.make_decode(wl)
    say("mfma decode window", window)
    out = from_dev(DecodeRun(inp).run(window=window))
    rows, want = oracle_decode_rows(inp, window=window)
    check_close(gpu_rows(out, rows, "bf16"), want, BF16_TOL, f"G=32 window {window}")


def test_large_group_decode_paged():
    wl = W.WORKLOADS["paged_long_decode"].replace(B=4, H=64, K=1, ctx=("loguniform", 30, 4000))
    inp = W.make_decode(wl)
    say("mfma decode paged G=64")
    out = from_dev(DecodeRun(inp).run())
    rows, want = oracle_decode_rows(inp)
    check_close(gpu_rows(out, rows, "bf16"), want, BF16_TOL, "paged G=64")


@pytest.mark.parametrize("H,K", [(64, 4), (64, 2), (64, 1), (66, 2)])
def test_large_group_id_is_exact(H, K):
    """V of KV head g is the constant g: every head h of group h // G returns g
    exactly (G = 64 and 32 and 33: split into two items, the 32-row and the
    64-row kernel)."""
    wl = LLAMA70.replace(B=3, H=H, K=K, ctx=("uniform", 20, 900))
    inp = W.make_decode(wl)
    for g in range(wl.K):
        inp.v[:, g] = W.f32_to_bf16_bits(np.float32([g]))[0]
    say("mfma decode group id", f"H={H} K={K}")
    out = as_f64(from_dev(DecodeRun(inp).run()), "bf16")
    G = wl.H // wl.K
    for h in range(wl.H):
        assert np.all(out[:, 0, h] == h // G), f"head {h}"


def _multi_case(wl, s, what, window=0, seqs=None):
    inp = W.make_decode(wl)
    run = DecodeRun(inp)
    rng = np.random.default_rng(wl.seed + 77)
    q = W.f32_to_bf16_bits(rng.standard_normal((wl.B, s, wl.H, wl.d)).astype(np.float32))
    say("decode multi", what, f"s={s} window={window}")
    out = binding.gqa_decode_multi(to_dev(q), run.cache, run.ctx, run.max_ctx, scale=wl.scale, window=window)
    torch.cuda.synchronize()
    o = from_dev(out)
    seqs = range(wl.B) if seqs is None else seqs
    got, want = [], []
    for b in seqs:
        n = int(inp.ctx[b])
        if inp.block_table is None:
            kb, vb = inp.k[b:b + 1, :, :n], inp.v[b:b + 1, :, :n]
        else:
            fill = W.sentinel(wl.dtype, "nan")
            kb = oracle.gather_paged_raw(inp.k, inp.block_table[b:b + 1], inp.ctx[b:b + 1], n, fill)
            vb = oracle.gather_paged_raw(inp.v, inp.block_table[b:b + 1], inp.ctx[b:b + 1], n, fill)
        rows = np.array([[0, i, h] for i in range(s) for h in range(wl.H)], dtype=np.int32)
        want.append(oracle.attention_rows(as_f64(q[b:b + 1], "bf16"), as_f64(kb, "bf16"), as_f64(vb, "bf16"),
                                          [n - s], [n], True, wl.scale, rows, window))
        got.append(as_f64(o[b][rows[:, 1], rows[:, 2]], "bf16"))
    check_close(np.concatenate(got), np.concatenate(want), BF16_TOL, f"decode multi {what}")


LLAMA3 = W.WORKLOADS["llama3_8b_decode"]


@pytest.mark.parametrize("s,H,K", [(2, 32, 8), (4, 32, 8), (8, 32, 8), (8, 64, 8), (4, 64, 4), (3, 24, 8),
                                   (2, 8, 8), (16, 32, 8), (16, 24, 8), (5, 40, 4)])
def test_decode_multi_matches_causal_oracle(s, H, K):
    wl = LLAMA3.replace(B=5, H=H, K=K, ctx=("uniform", 16, 1200))
    _multi_case(wl, s, f"H={H} K={K}")


@pytest.mark.parametrize("window", [1, 3, 300])
def test_decode_multi_window(window):
    _multi_case(LLAMA3.replace(B=4, ctx=("uniform", 20, 1500)), 4, f"window {window}", window=window)


def test_decode_multi_paged():
    wl = W.WORKLOADS["paged_long_decode"].replace(B=4, H=32, K=8, ctx=("loguniform", 20, 3000))
    _multi_case(wl, 8, "paged")


def test_decode_multi_whole_context_is_new():
    """ctx == s: the block is the whole sequence, a plain causal prefill of s rows."""
    inp_wl = LLAMA3.replace(B=3, ctx=("fixed", 8))
    _multi_case(inp_wl, 8, "ctx == s")


def test_decode_multi_full_size_sampled():
    _multi_case(LLAMA3, 4, "llama3_8b_decode shape, s=4", seqs=[0, 17, 31])


def test_decode_multi_rejects_unsupported():
    wl = LLAMA3.replace(B=2, ctx=("uniform", 20, 40))
    inp = W.make_decode(wl)
    run = DecodeRun(inp)
    q = to_dev(W.f32_to_bf16_bits(np.zeros((2, 17, wl.H, wl.d), dtype=np.float32)))   # 17 * 4 > 64 rows
    with pytest.raises(binding.GqaError):
        binding.gqa_decode_multi(q, run.cache, run.ctx, run.max_ctx)
