"""The whole decode step in one call (gqa_decode_step): append the newest
token's K/V and attend, against the two-call form (gqa_kv_append, then
gqa_decode_window) and against the oracle.

The concept page's technical principle (技术原理) has each new token's K/V
join the cache before its query attends to the cached keys; the one-call form
must leave exactly the cache bytes the append leaves and give exactly the
output the two calls give (the same kernel arithmetic on the same values).
To show that the fused kernel takes the new token from k_new / v_new and
not from the cache, the cache slot it is about to fill holds NaN before the
call."""
import numpy as np
import pytest
import torch

from grouped_query_attention_gqa_amd import binding
from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import (BF16_TOL, F32_TOL, check_close, from_dev, gpu_rows, oracle_decode_rows, say, to_dev)

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _poison_new_slots(inp: W.DecodeInputs, k: np.ndarray, v: np.ndarray):
    """Copies of the cache arrays with each sequence's slot ctx - 1 set to NaN."""
    k, v = k.copy(), v.copy()
    nan = W.sentinel(inp.wl.dtype, "nan")
    for b in range(inp.wl.B):
        t = int(inp.ctx[b]) - 1
        if inp.block_table is None:
            k[b, :, t] = nan
            v[b, :, t] = nan
        else:
            blk = int(inp.block_table[b, t // inp.wl.block_size])
            k[blk, :, t % inp.wl.block_size] = nan
            v[blk, :, t % inp.wl.block_size] = nan
    return k, v


def _step_case(wl: W.Workload, what: str, window: int = 0, seqs=None):
    inp = W.make_decode(wl)
    kn, vn = inp.new_token_rows()
    k0, v0 = _poison_new_slots(inp, inp.k, inp.v)
    bt = None if inp.block_table is None else to_dev(inp.block_table)
    q, ctx = to_dev(inp.q), to_dev(inp.ctx)
    kn_d, vn_d = to_dev(kn), to_dev(vn)
    max_ctx = int(inp.ctx.max())
    tol = BF16_TOL if wl.dtype == "bf16" else F32_TOL

    say("decode step (one call)", what, f"window={window}")
    c1 = binding.KVCache(to_dev(k0), to_dev(v0), bt)
    out1 = binding.gqa_decode_step(q, kn_d, vn_d, c1, ctx, max_ctx, scale=wl.scale, window=window)
    torch.cuda.synchronize()

    say("decode step (append, then decode)", what, f"window={window}")
    c2 = binding.KVCache(to_dev(k0), to_dev(v0), bt)
    start = to_dev((inp.ctx - 1).astype(np.int32))
    binding.gqa_kv_append(c2, kn_d, vn_d, start)
    out2 = binding.gqa_decode(q, c2, ctx, max_ctx, scale=wl.scale, window=window)
    torch.cuda.synchronize()

    # the same output bits and the same cache bytes (NaN slots compared as bytes)
    o1, o2 = from_dev(out1), from_dev(out2)
    assert o1.view(np.uint8).tobytes() == o2.view(np.uint8).tobytes(), f"{what}: outputs differ"
    for name, a, b in (("k", c1.k, c2.k), ("v", c1.v, c2.v)):
        assert from_dev(a).view(np.uint8).tobytes() == from_dev(b).view(np.uint8).tobytes(), \
            f"{what}: cache {name} differs"
    # the step put back exactly the rows the poisoned slots held
    assert from_dev(c1.k).view(np.uint8).tobytes() == np.ascontiguousarray(inp.k).view(np.uint8).tobytes(), \
        f"{what}: cache k after the step is not the appended cache"
    assert from_dev(c1.v).view(np.uint8).tobytes() == np.ascontiguousarray(inp.v).view(np.uint8).tobytes(), \
        f"{what}: cache v after the step is not the appended cache"
    rows, want = oracle_decode_rows(inp, seqs=seqs, window=window)
    check_close(gpu_rows(o1, rows, wl.dtype), want, tol, f"decode step {what}")


LLAMA3 = W.WORKLOADS["llama3_8b_decode"]


# G = 4, 8, 1, 2; G = 32 (the 32-row kernel), 64 (two items of 32 heads) and
# 33 (the 64-row kernel)
@pytest.mark.parametrize("H,K", [(32, 8), (64, 8), (16, 16), (16, 8), (64, 64), (32, 1), (64, 1), (66, 2)])
def test_step_matches_append_then_decode_bf16(H, K):
    wl = LLAMA3.replace(B=6, H=H, K=K, ctx=("uniform", 1, 700))
    _step_case(wl, f"bf16 H={H} K={K}")


def test_step_ctx_one_and_tile_edges():
    # contexts at 1 and at the edges of 32-key tiles and 16-key groups
    lens = [1, 16, 17, 31, 32, 33, 64, 65]
    inp = W.make_decode(LLAMA3.replace(B=len(lens), ctx=("uniform", 1, 65)), ctx_override=lens)
    _step_case_inputs(inp, "ctx edges")


def _step_case_inputs(inp: W.DecodeInputs, what: str, window: int = 0):
    wl = inp.wl
    kn, vn = inp.new_token_rows()
    k0, v0 = _poison_new_slots(inp, inp.k, inp.v)
    bt = None if inp.block_table is None else to_dev(inp.block_table)
    q, ctx = to_dev(inp.q), to_dev(inp.ctx)
    say("decode step (one call)", what)
    c1 = binding.KVCache(to_dev(k0), to_dev(v0), bt)
    out1 = binding.gqa_decode_step(q, to_dev(kn), to_dev(vn), c1, ctx, int(inp.ctx.max()), scale=wl.scale,
                                   window=window)
    torch.cuda.synchronize()
    assert from_dev(c1.k).view(np.uint8).tobytes() == np.ascontiguousarray(inp.k).view(np.uint8).tobytes()
    assert from_dev(c1.v).view(np.uint8).tobytes() == np.ascontiguousarray(inp.v).view(np.uint8).tobytes()
    rows, want = oracle_decode_rows(inp, window=window)
    check_close(gpu_rows(from_dev(out1), rows, wl.dtype), want, BF16_TOL, f"decode step {what}")


@pytest.mark.parametrize("window", [1, 5, 100])
def test_step_with_window(window):
    _step_case(LLAMA3.replace(B=5, ctx=("uniform", 1, 900)), f"window {window}", window=window)


@pytest.mark.parametrize("block_size", [16, 64, 4])
def test_step_paged(block_size):
    wl = W.WORKLOADS["paged_long_decode"].replace(B=5, ctx=("loguniform", 20, 3000), block_size=block_size)
    _step_case(wl, f"paged bs={block_size}", seqs=[0, 2, 4])


def test_step_paged_large_group():
    wl = W.WORKLOADS["paged_long_decode"].replace(B=4, H=64, K=1, ctx=("loguniform", 20, 3000), block_size=16)
    _step_case(wl, "paged G=64", seqs=[0, 1, 3])


def test_step_fp32_appends_first():
    wl = W.WORKLOADS["tiny_decode_f32"]
    _step_case(wl, "fp32")


def test_step_full_size_llama3():
    # the workload the bench times: sampled rows against the oracle
    _step_case(LLAMA3, "llama3_8b_decode", seqs=[0, 7, 31])
