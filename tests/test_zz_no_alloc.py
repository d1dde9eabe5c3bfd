"""gqa_decode_step_noalloc: the decode step with the library's static
workspace (for callers that cannot allocate) against gqa_decode_step with a
caller's workspace, through the C ABI.

Both run the same kernels, so the outputs and the cache bytes must be
identical; the output must also meet the oracle's tolerance.  Two calls in a
row, the second on a smaller input, check that the buffer's leftovers from
the first call do not leak into the second.
"""
import numpy as np
import pytest
import torch

from grouped_query_attention_gqa_amd import binding
from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import BF16_TOL, F32_TOL, check_close, from_dev, gpu_rows, oracle_decode_rows, requires_gpu, say, to_dev

pytestmark = [pytest.mark.gpu, requires_gpu]


class Case:
    def __init__(self, wl, ctx=None):
        self.inp = W.make_decode(wl, ctx_override=ctx)
        self.wl = wl
        kn, vn = self.inp.new_token_rows()
        self.kn, self.vn = to_dev(kn), to_dev(vn)
        self.q = to_dev(self.inp.q)
        self.ctx = to_dev(self.inp.ctx)
        self.max_ctx = int(self.inp.ctx.max())
        self.bt = None if self.inp.block_table is None else to_dev(self.inp.block_table)

    def cache(self):
        """A fresh device copy of the cache, with each newest row cleared so that
        the step's own write of it is what the attention reads."""
        k, v = self.inp.k.copy(), self.inp.v.copy()
        for b in range(self.wl.B):
            t = int(self.inp.ctx[b]) - 1
            if self.inp.block_table is None:
                k[b, :, t] = 0
                v[b, :, t] = 0
            else:
                blk = int(self.inp.block_table[b, t // self.wl.block_size])
                k[blk, :, t % self.wl.block_size] = 0
                v[blk, :, t % self.wl.block_size] = 0
        return binding.KVCache(to_dev(k), to_dev(v), self.bt)

    def run(self, noalloc, step=True):
        cache = self.cache()
        out = torch.full_like(self.q, 3.0)
        kn, vn = (self.kn, self.vn) if step else (None, None)
        if noalloc:
            binding.gqa_decode_step_noalloc(self.q, kn, vn, cache, self.ctx, self.max_ctx, out=out, scale=self.wl.scale)
        elif step:
            binding.gqa_decode_step(self.q, kn, vn, cache, self.ctx, self.max_ctx, out=out, scale=self.wl.scale)
        torch.cuda.synchronize()
        return from_dev(out), from_dev(cache.k), from_dev(cache.v)


def _compare(case, what):
    say("noalloc", what)
    got, gk, gv = case.run(True)
    want, wk, wv = case.run(False)
    assert got.tobytes() == want.tobytes(), f"{what}: output differs from gqa_decode_step"
    assert gk.tobytes() == wk.tobytes() and gv.tobytes() == wv.tobytes(), f"{what}: cache differs"
    rows, ref = oracle_decode_rows(case.inp)
    tol = F32_TOL if case.wl.dtype == "f32" else BF16_TOL
    check_close(gpu_rows(got, rows, case.wl.dtype), ref, tol, what)


def test_noalloc_step_matches_the_workspace_call_twice_in_a_row():
    big = Case(W.WORKLOADS["llama3_8b_decode"])                                   # the full Llama-3-8B step
    small = Case(W.WORKLOADS["llama3_8b_decode"].replace(B=3, ctx=("uniform", 1, 700)), ctx=[700, 1, 33])
    _compare(big, "llama3_8b_decode, full size")
    _compare(small, "smaller input after it")


def test_noalloc_step_other_kernels_and_paged():
    _compare(Case(W.WORKLOADS["paged_long_decode"].replace(B=6, ctx=("loguniform", 100, 6000))), "paged, G = 8")
    _compare(Case(W.WORKLOADS["llama3_8b_decode"].replace(B=5, d=64, ctx=("uniform", 1, 900))), "d = 64")
    _compare(Case(W.WORKLOADS["tiny_decode_f32"].replace(B=2)), "fp32")


def test_noalloc_plain_decode_equals_gqa_decode():
    case = Case(W.WORKLOADS["llama3_8b_decode"].replace(B=4, ctx=("uniform", 1, 2000)))
    cache = binding.KVCache(to_dev(case.inp.k), to_dev(case.inp.v))
    say("noalloc plain decode")
    a = binding.gqa_decode_step_noalloc(case.q, None, None, cache, case.ctx, case.max_ctx, scale=case.wl.scale)
    b = binding.gqa_decode(case.q, cache, case.ctx, case.max_ctx, scale=case.wl.scale)
    torch.cuda.synchronize()
    assert from_dev(a).tobytes() == from_dev(b).tobytes()


def test_noalloc_refuses_a_call_beyond_its_buffer():
    """G = 64 at d = 128 needs ~33 MiB of partials: more than the 12 MiB buffer."""
    wl = W.WORKLOADS["llama2_70b_decode_mqa"].replace(B=2, ctx=("fixed", 64))
    case = Case(wl)
    cache = case.cache()
    out = torch.full_like(case.q, 3.0)
    say("noalloc too large")
    with pytest.raises(binding.GqaError) as e:
        binding.gqa_decode_step_noalloc(case.q, case.kn, case.vn, cache, case.ctx, case.max_ctx, out=out)
    assert e.value.status == binding.GQA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert (out == 3.0).all()
