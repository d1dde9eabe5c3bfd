"""GPU parity over a seeded random sweep of shapes, against the fp64 oracle.

Each case draws its own head counts, context lengths (ragged, exact tile
multiples, a single key), cache layout (contiguous, or paged with 16- to
128-token blocks dealt at random), sliding window and, for the prefill, the
cached prefix, the chunk length and causal or full attention.  The case list
is fixed by its seed; every output row is compared (bf16 tolerance 2e-2),
and the bf16 prefill's cache bytes must equal the oracle's append.  The
sweep reaches the decode kernel's uniform fast paths (whole visible tiles,
tiles inside every row's window) and their edges, and the FP8 (and INT8) prefill's
steady and masked tile code; the fused decode step and the decode of several
newest positions per sequence draw their shapes the same way."""
import numpy as np
import pytest

from grouped_query_attention_gqa_amd import workloads as W
from gpu_common import (BF16_TOL, DecodeRun, PrefillRun, check_close, from_dev, gpu_rows, oracle_decode_rows,
                        oracle_prefill_rows, requires_gpu, say)

pytestmark = [pytest.mark.gpu, requires_gpu]

HEADS = [(32, 8), (64, 8), (16, 16), (64, 1), (24, 8), (8, 2), (48, 3), (64, 4)]


def _draw_ctx(rng, B, hi):
    """Context lengths mixing the edges of a 16-key tile with random lengths."""
    picks = []
    for _ in range(B):
        kind = rng.integers(0, 4)
        if kind == 0:
            picks.append(1)
        elif kind == 1:
            picks.append(16 * int(rng.integers(1, hi // 16 + 1)))
        elif kind == 2:
            picks.append(16 * int(rng.integers(0, hi // 16)) + int(rng.integers(1, 16)))
        else:
            picks.append(int(rng.integers(1, hi + 1)))
    return picks


def _decode_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        H, K = HEADS[rng.integers(0, len(HEADS))]
        B = int(rng.integers(1, 6))
        ctx = _draw_ctx(rng, B, 900)
        paged = bool(rng.integers(0, 2))
        bs = int(rng.choice([16, 32, 64, 128]))
        window = 0 if rng.integers(0, 2) == 0 else int(rng.integers(1, 400))
        cases.append(dict(i=i, H=H, K=K, B=B, ctx=ctx, paged=paged, bs=bs, window=window,
                          seed=int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _decode_cases(40, 20261202), ids=lambda c: f"decode{c['i']}")
def test_decode_sweep(case):
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=case["B"], H=case["H"], K=case["K"], seed=case["seed"],
                                                ctx=("uniform", 1, 900), paged=case["paged"],
                                                block_size=case["bs"])
    inp = W.make_decode(wl, ctx_override=case["ctx"])
    what = f"decode sweep {case}"
    say(what)
    out = from_dev(DecodeRun(inp).run(window=case["window"]))
    rows, want = oracle_decode_rows(inp, window=case["window"])
    check_close(gpu_rows(out, rows, "bf16"), want, BF16_TOL, what)


def _prefill_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        H, K = HEADS[rng.integers(0, len(HEADS))]
        B = int(rng.integers(1, 4))
        s = int(rng.choice([1, 7, 64, 65, int(rng.integers(2, 130))]))
        start = int(rng.choice([0, 0, 64, int(rng.integers(1, 400))]))
        paged = bool(rng.integers(0, 2))
        bs = int(rng.choice([16, 32, 64]))
        causal = bool(rng.integers(0, 4) != 0)
        window = 0 if (not causal or rng.integers(0, 2) == 0) else int(rng.integers(1, 300))
        cases.append(dict(i=i, H=H, K=K, B=B, s=s, start=start, paged=paged, bs=bs, causal=causal, window=window,
                          seed=int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("case", _prefill_cases(40, 31337), ids=lambda c: f"prefill{c['i']}")
def test_prefill_sweep(case):
    wl = W.WORKLOADS["causal_prefill_4k"].replace(B=case["B"], s=case["s"], H=case["H"], K=case["K"],
                                                 seed=case["seed"], block_size=case["bs"])
    base = W.make_prefill(wl)
    rng = np.random.default_rng(case["seed"])
    P = case["start"]
    starts = np.full(wl.B, P, np.int32)
    inp = W.PrefillInputs(wl, starts, base.q, base.k_new, base.v_new)
    prior = None
    if P > 0:
        bits = lambda shape: W.f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
        prior = (bits((wl.B, P, wl.K, wl.d)), bits((wl.B, P, wl.K, wl.d)))
    paged_blocks = None
    if case["paged"]:
        paged_blocks = W.deal_blocks(rng, starts + wl.s, wl.block_size, slack_blocks=3)
    what = f"prefill sweep {case}"
    say(what)
    run = PrefillRun(inp, paged_blocks=paged_blocks, prior=prior)
    out = from_dev(run.run(causal=case["causal"], window=case["window"]))
    run.check_cache(what)
    rows = np.array([[b, i, h] for b in range(wl.B) for i in range(wl.s) for h in range(wl.H)], np.int32)
    want = oracle_prefill_rows(inp, rows, causal=case["causal"], prior=prior, window=case["window"])
    check_close(gpu_rows(out, rows, "bf16"), want, BF16_TOL, what)


@pytest.mark.parametrize("case", _decode_cases(20, 777), ids=lambda c: f"fp8decode{c['i']}")
def test_fp8_decode_sweep(case):
    from test_fp8_gpu import _decode_case as fp8_decode_case
    # (the FP8 helper draws the contexts from the workload's seed)
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=case["B"], H=case["H"], K=case["K"], seed=case["seed"],
                                                ctx=("uniform", 1, 900), paged=case["paged"], block_size=case["bs"])
    fp8_decode_case(wl, f"sweep {case}", window=case["window"])


@pytest.mark.parametrize("case", _prefill_cases(20, 4242), ids=lambda c: f"fp8prefill{c['i']}")
def test_fp8_prefill_sweep(case):
    from test_fp8_gpu import _check_fp8_prefill
    _check_fp8_prefill(f"fp8 prefill sweep {case}", B=case["B"], H=case["H"], K=case["K"], s=case["s"],
                       start=case["start"], paged=case["paged"], bs=case["bs"], causal=case["causal"],
                       window=case["window"], seed=case["seed"])


@pytest.mark.parametrize("case", _decode_cases(20, 8888), ids=lambda c: f"int8decode{c['i']}")
def test_int8_decode_sweep(case):
    from test_fp8_gpu import _decode_case as q_decode_case
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=case["B"], H=case["H"], K=case["K"], seed=case["seed"],
                                                ctx=("uniform", 1, 900), paged=case["paged"], block_size=case["bs"])
    q_decode_case(wl, f"sweep {case}", window=case["window"], codec="int8")


@pytest.mark.parametrize("case", _prefill_cases(20, 5353), ids=lambda c: f"int8prefill{c['i']}")
def test_int8_prefill_sweep(case):
    from test_fp8_gpu import _check_fp8_prefill
    _check_fp8_prefill(f"int8 prefill sweep {case}", B=case["B"], H=case["H"], K=case["K"], s=case["s"],
                       start=case["start"], paged=case["paged"], bs=case["bs"], causal=case["causal"],
                       window=case["window"], seed=case["seed"], codec="int8")



# the fused decode step (append of the newest token + decode, checked against
# append-then-decode bit for bit and against the oracle) and the decode of
# several newest positions per sequence (s * G <= 64 rows per KV head)
@pytest.mark.parametrize("case", _decode_cases(16, 6060), ids=lambda c: f"step{c['i']}")
def test_step_sweep(case):
    from test_decode_step_gpu import _step_case
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=case["B"], H=case["H"], K=case["K"], seed=case["seed"],
                                                ctx=("uniform", 1, 900), paged=case["paged"], block_size=case["bs"])
    _step_case(wl, f"sweep {case}", window=case["window"])


def _multi_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for c in _decode_cases(n, seed):
        if c["H"] // c["K"] > 32:
            c["H"], c["K"] = 32, 1
        G = c["H"] // c["K"]
        c["s"] = int(rng.integers(2, 64 // G + 1))
        cases.append(c)
    return cases


@pytest.mark.parametrize("case", _multi_cases(16, 7070), ids=lambda c: f"multi{c['i']}")
def test_multi_sweep(case):
    from test_decode_multi_gpu import _multi_case
    wl = W.WORKLOADS["llama3_8b_decode"].replace(B=case["B"], H=case["H"], K=case["K"], seed=case["seed"],
                                                ctx=("uniform", 16, 900), paged=case["paged"], block_size=case["bs"])
    _multi_case(wl, case["s"], f"sweep {case}", window=case["window"])

# ---------------------------------------------------------------------------
# the other shapes: bf16 at d = 64 (the matrix-core decode's and prefill's
# d = 64 code) and fp32 at d = 64 and 128 (the row-streaming kernel)
# ---------------------------------------------------------------------------

def _other_cases(n, seed, kind):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        H, K = HEADS[rng.integers(0, len(HEADS))]
        dtype, d = [("bf16", 64), ("f32", 64), ("f32", 128)][rng.integers(0, 3)]
        paged = dtype == "bf16" and bool(rng.integers(0, 2))
        c = dict(i=i, H=H, K=K, dtype=dtype, d=d, paged=paged, bs=int(rng.choice([16, 32, 64])),
                 seed=int(rng.integers(1 << 30)))
        if kind == "decode":
            c.update(B=int(rng.integers(1, 5)), window=0 if rng.integers(0, 2) == 0 else int(rng.integers(1, 300)))
            c["ctx"] = _draw_ctx(rng, c["B"], 600)
        else:
            c.update(B=int(rng.integers(1, 3)), s=int(rng.choice([1, 33, 64, int(rng.integers(2, 100))])),
                     causal=bool(rng.integers(0, 4) != 0))
            c["window"] = 0 if (not c["causal"] or rng.integers(0, 2) == 0) else int(rng.integers(1, 200))
        cases.append(c)
    return cases


def _tol(dtype):
    from gpu_common import F32_TOL
    return BF16_TOL if dtype == "bf16" else F32_TOL


@pytest.mark.parametrize("case", _other_cases(30, 99, "decode"),
                         ids=lambda c: f"decode_{c['dtype']}_d{c['d']}_{c['i']}")
def test_other_decode_sweep(case):
    base = W.WORKLOADS["llama3_8b_decode"] if case["dtype"] == "bf16" else W.WORKLOADS["tiny_decode_f32"]
    wl = base.replace(B=case["B"], H=case["H"], K=case["K"], d=case["d"], seed=case["seed"],
                      ctx=("uniform", 1, 600), paged=case["paged"], block_size=case["bs"])
    inp = W.make_decode(wl, ctx_override=case["ctx"])
    what = f"decode sweep {case}"
    say(what)
    out = from_dev(DecodeRun(inp).run(window=case["window"]))
    rows, want = oracle_decode_rows(inp, window=case["window"])
    check_close(gpu_rows(out, rows, case["dtype"]), want, _tol(case["dtype"]), what)


@pytest.mark.parametrize("case", _other_cases(30, 1234, "prefill"), ids=lambda c: f"prefill_{c['dtype']}_d{c['d']}_{c['i']}")
def test_other_prefill_sweep(case):
    base = W.WORKLOADS["causal_prefill_4k"] if case["dtype"] == "bf16" else W.WORKLOADS["tiny_prefill_f32"]
    wl = base.replace(B=case["B"], s=case["s"], H=case["H"], K=case["K"], d=case["d"], seed=case["seed"],
                      block_size=case["bs"])
    inp = W.make_prefill(wl)
    rng = np.random.default_rng(case["seed"])
    paged_blocks = W.deal_blocks(rng, inp.start_pos + wl.s, wl.block_size, slack_blocks=2) if case["paged"] else None
    what = f"prefill sweep {case}"
    say(what)
    run = PrefillRun(inp, paged_blocks=paged_blocks)
    out = from_dev(run.run(causal=case["causal"], window=case["window"]))
    run.check_cache(what)
    rows = np.array([[b, i, h] for b in range(wl.B) for i in range(wl.s) for h in range(wl.H)], np.int32)
    want = oracle_prefill_rows(inp, rows, causal=case["causal"], window=case["window"])
    check_close(gpu_rows(out, rows, case["dtype"]), want, _tol(case["dtype"]), what)
