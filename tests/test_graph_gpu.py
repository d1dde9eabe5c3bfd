"""The library's calls inside HIP graphs.

The calls launch kernels on the caller's stream and nothing else (no
allocation, no memset, no host synchronisation), so a caller may capture
them.  Each graph here is replayed several times, with eager work and
synchronisations between the replays, and every replay must give the eager
call's output bit for bit."""
import numpy as np
import pytest
import torch

from grouped_query_attention_gqa_amd import binding
from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import from_dev, say, to_dev

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _replays_match(call, out: torch.Tensor, what: str, replays: int = 3):
    say("graph", what, "eager")
    call()
    torch.cuda.synchronize()
    want = from_dev(out).copy()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    say("graph", what, "capture")
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device="cuda")
    for r in range(replays):
        out.fill_(0)                      # eager work between replays
        scratch.mul_(1.0001).add_(0.5)
        torch.cuda.synchronize()
        say("graph", what, f"replay {r}")
        g.replay()
        torch.cuda.synchronize()
        got = from_dev(out)
        assert got.view(np.uint8).tobytes() == want.view(np.uint8).tobytes(), f"{what}: replay {r} differs"
    del g


@pytest.mark.parametrize("name", ["llama3_8b_decode", "paged_long_decode", "llama2_70b_decode_mqa"])
def test_decode_step_in_a_graph(name):
    wl = W.WORKLOADS[name].replace(B=6, ctx=("uniform", 40, 3000))
    inp = W.make_decode(wl)
    kn, vn = inp.new_token_rows()
    q, ctx, kn, vn = to_dev(inp.q), to_dev(inp.ctx), to_dev(kn), to_dev(vn)
    bt = None if inp.block_table is None else to_dev(inp.block_table)
    cache = binding.KVCache(to_dev(inp.k), to_dev(inp.v), bt)
    out = torch.empty_like(q)
    ws = torch.zeros(binding.gqa_decode_workspace_bytes(wl.B, wl.H, wl.K, wl.d, int(inp.ctx.max())),
                     dtype=torch.uint8, device="cuda")
    m = int(inp.ctx.max())
    _replays_match(lambda: binding.gqa_decode_step(q, kn, vn, cache, ctx, m, out=out, scale=wl.scale, workspace=ws),
                   out, f"decode step {name}")
    _replays_match(lambda: binding.gqa_decode(q, cache, ctx, m, out=out, scale=wl.scale, workspace=ws, window=100),
                   out, f"decode window {name}")


def test_prefill_in_a_graph():
    wl = W.WORKLOADS["chunked_prefill_paged"].replace(B=2, s=200, start=300)
    inp = W.make_prefill(wl)
    q, kn, vn, start = to_dev(inp.q), to_dev(inp.k_new), to_dev(inp.v_new), to_dev(inp.start_pos)
    S = wl.start + wl.s
    nblk = (S + wl.block_size - 1) // wl.block_size
    table = np.arange(wl.B * nblk, dtype=np.int32)[::-1].copy().reshape(wl.B, nblk)
    shape = (wl.B * nblk, wl.K, wl.block_size, wl.d)
    k = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
    v = torch.zeros_like(k)
    cache = binding.KVCache(k, v, to_dev(table))
    out = torch.empty_like(q)
    _replays_match(lambda: binding.gqa_prefill(q, kn, vn, cache, start, causal=True, out=out, scale=wl.scale),
                   out, "chunked paged prefill")


def test_fp8_prefill_and_noalloc_step_in_a_graph():
    """The FP8-cache prefill (append + prefill kernels) and the decode step with
    the library's static workspace, captured and replayed."""
    wl = W.WORKLOADS["chunked_prefill_paged"].replace(B=2, s=130, start=200)
    inp = W.make_prefill(wl)
    q, kn, vn, start = to_dev(inp.q), to_dev(inp.k_new), to_dev(inp.v_new), to_dev(inp.start_pos)
    S = wl.start + wl.s
    k = torch.zeros((wl.B, wl.K, S, wl.d), dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    v = torch.zeros_like(k)
    ks = torch.zeros((wl.B, wl.K, S), dtype=torch.float32, device="cuda")
    cache = binding.KVCache(k, v, None, k_scale=ks, v_scale=torch.zeros_like(ks))
    out = torch.empty_like(q)
    _replays_match(lambda: binding.gqa_prefill(q, kn, vn, cache, start, causal=True, out=out, scale=wl.scale),
                   out, "fp8 prefill")
    dw = W.WORKLOADS["llama3_8b_decode"].replace(B=5, ctx=("uniform", 40, 2000))
    dinp = W.make_decode(dw)
    dkn, dvn = dinp.new_token_rows()
    dq, dctx, dkn, dvn = to_dev(dinp.q), to_dev(dinp.ctx), to_dev(dkn), to_dev(dvn)
    dcache = binding.KVCache(to_dev(dinp.k), to_dev(dinp.v))
    dout = torch.empty_like(dq)
    m = int(dinp.ctx.max())
    _replays_match(lambda: binding.gqa_decode_step_noalloc(dq, dkn, dvn, dcache, dctx, m, out=dout, scale=dw.scale),
                   dout, "decode step, static workspace")
