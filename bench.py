#!/usr/bin/env python3
"""Benchmark of the grouped-query attention hot path on one MI355X.

A step is one decode step of the Llama-3-8B-shaped workload (B=32, H=32,
K=8, d=128, bf16, contexts drawn from U[1024, 4096]): gqa_decode_step, which
appends every sequence's newest token and attends over the whole cache in
one call.  `value` is the step's algorithmic bytes (the K/V rows every query
must read once, plus Q, O and the appended rows) divided by the step time,
in GB/s.

The same JSON line also carries
  * roofline: the decode step's kernels (HBM bound), timed with HIP events on
    the stream they run on, against MI355X's 8 TB/s; two_call_step: the same
    step as gqa_kv_append followed by gqa_decode, for comparison;
  * prefill: the causal prefill workload (B=4, s=4096, H=32, K=8, d=128,
    bf16, append included) in TFLOP/s against the 2.5 PFLOP/s dense bf16
    matrix-core peak;
  * decode_workloads: the other decode shapes (Llama-2-70B contiguous and its
    MHA / MQA variants, paged long-context, a Mistral-7B-shaped
    sliding-window decode whose bytes count only the window, and the
    Llama-3-8B decode on an FP8 E4M3 cache with a scale per row, whose bytes
    are the codes and scales, and the same shape with four new positions per
    sequence decoded at once by gqa_decode_multi) in GB/s;
  * prefill_workloads: a chunked prefill (512 new tokens after a 3584-token
    cached prefix, paged cache) in TFLOP/s, on a bf16 cache and on an FP8
    E4M3 cache with a scale per row;
  * tiny_workloads: the two tiny fp32 workloads (causal prefill of 128
    tokens, decode over 128 cached tokens) in microseconds per call;
  * cpu_baseline: the CPU oracle on the host cores, on the same step, with
    the host's CPU model; its `workloads` entry times the oracle on bounded
    samples of the other workloads (decode GB/s, prefill GFLOP/s, tiny-call
    microseconds);
  * pages_context: the pages' own figures with the hardware they were
    measured on (context only, not targets).

The K/V caches are rotated over several copies so that the ~256 MB
Infinity Cache cannot serve them between steps; inputs are resident in HBM
before the timed region starts.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# gqa_decode is the main kernel plus the small merge of cut items; events time both
DECODE_KERNELS = ("decode_mfma_kernel<1, false> (with the append of the newest token) + merge_rows_kernel "
                  "(one gqa_decode_step call)")
DECODE_SOURCES = ("decode_mfma.hip", "stream_attention.hip", "worklist.h", "kernels.h", "common.h")
PREFILL_SOURCES = ("prefill_mfma.hip", "kv_append.hip", "kernels.h", "common.h")
PREFILL_FP8_SOURCES = ("prefill_fp8.hip", "kv_append.hip", "kernels.h", "common.h")
# the kernel sources each committed byte-counter figure was taken on
TRAFFIC_SOURCES = {
    "decode/llama3_8b_decode": DECODE_SOURCES,
    "decode/llama2_70b_decode": DECODE_SOURCES,
    "decode/paged_long_decode": DECODE_SOURCES,
    "decode/llama2_70b_decode_mqa": DECODE_SOURCES,
    "decode/llama3_8b_decode_fp8_cache": DECODE_SOURCES + ("kv_append.hip",),
    "decode/llama3_8b_decode_int8_cache": DECODE_SOURCES + ("kv_append.hip",),
    "prefill/causal_prefill_4k": PREFILL_SOURCES,
    "prefill/chunked_prefill_paged_fp8_cache": PREFILL_FP8_SOURCES,
    "prefill/chunked_prefill_paged_int8_cache": PREFILL_FP8_SOURCES,
}
BF16_MFMA_PEAK_TFLOPS = 2500.0
METRIC = "GQA decode HBM GB/s (% of peak) + causal prefill TFLOP/s (% MFMA peak), bf16"
MALL_BYTES = 256 * 2**20
COPY_BYTES = 512 * 2**20   # calibration copy for the HBM byte counters
LEG_CALLS = 50             # timed calls of every leg beside the headline, whatever --steps is


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="only the headline decode step")
    ap.add_argument("--only", default=None,
                    help="profile one kernel: decode|step|fp8|int8|multi|prefill|decode70b|paged|mha|mqa|window|d64|chunked|"
                         "chunked_fp8|chunked_int8|"
                         "tiny_prefill|tiny_decode (both tiny fp32 workloads)|copy (a 512 MiB device copy)")
    ap.add_argument("--summarize", default=None, help="print the per-kernel summary of a rocprofv3 trace directory")
    ap.add_argument("--traffic", nargs=6, default=None,
                    metavar=("KEY", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR", "ALG_BYTES"),
                    help="record one leg's byte counters (rocprofv3 --pmc runs) in profiles/traffic.json")
    return ap.parse_args()


# ---------------------------------------------------------------------------
# device helpers
# ---------------------------------------------------------------------------

def up(x: np.ndarray):
    import torch
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def decode_bytes(wl, ctx, fp8=False):
    """Algorithmic bytes of one decode: each visible K and V row once (with a
    sliding window only the window's rows), Q read, O written.  An FP8 cache
    row (or INT8) is d one-byte codes plus its 4-byte scale; Q and O stay
    bf16."""
    es = 2 if wl.dtype == "bf16" else 4
    rows = np.minimum(ctx, wl.window) if wl.window > 0 else ctx
    row_bytes = wl.d + 4 if fp8 else wl.d * es
    kv = 2 * wl.K * row_bytes * int(np.sum(rows, dtype=np.int64))
    qo = 2 * wl.B * wl.H * wl.d * es
    return kv + qo


def append_bytes(wl, s_new):
    es = 2 if wl.dtype == "bf16" else 4
    return 2 * 2 * wl.B * s_new * wl.K * wl.d * es   # K and V rows, read once and written once


def causal_flops(wl):
    """4 * B * H * d * sum_{i<s} (start+i+1): QK^T and PV over the visible keys (the
    cached prefix and the lower triangle of the new tokens)."""
    return 4 * wl.B * wl.H * wl.d * (wl.s * wl.start + wl.s * (wl.s + 1) // 2)


class DecodeBench:
    """Device-resident copies of one decode workload, rotated per call."""

    def __init__(self, wl, copies=None, fp8=False, mq=1, int8=False):
        import torch
        from grouped_query_attention_gqa_amd import binding
        from grouped_query_attention_gqa_amd import workloads as W
        self.wl = wl
        fp8 = fp8 or int8   # a 1-byte cache: the same bytes, INT8 codes with int8
        t0 = time.time()
        inp = W.make_decode(wl, fill="zero")
        self.inp = inp
        self.ctx = inp.ctx
        self.max_ctx = int(inp.ctx.max())
        self.alg_bytes = decode_bytes(wl, inp.ctx, fp8) + (mq - 1) * 2 * wl.B * wl.H * wl.d * 2   # q/out of mq rows
        self.mq = mq
        valid = self.alg_bytes
        n = copies if copies is not None else max(1, min(4, math.ceil(3 * MALL_BYTES / max(valid, 1))))
        self.q = up(inp.q)
        self.ctx_d = up(inp.ctx)
        kn, vn = inp.new_token_rows()
        self.k_new, self.v_new = up(kn), up(vn)
        self.start = up((inp.ctx - 1).astype(np.int32))
        self.caches = []
        k0, v0 = up(inp.k), up(inp.v)
        bt = None if inp.block_table is None else up(inp.block_table)
        if fp8:
            # the FP8 (INT8) cache is filled by the library's quantising append
            # of every cached position (contiguous caches)
            assert bt is None, "the quantised-cache bench legs use a contiguous cache"
            B, K, S, d = k0.shape
            kt, vt = k0.permute(0, 2, 1, 3).contiguous(), v0.permute(0, 2, 1, 3).contiguous()
            zero = torch.zeros(B, dtype=torch.int32, device="cuda")
            del k0, v0
            for i in range(n):
                kq = torch.empty((B, K, S, d), dtype=torch.uint8, device="cuda").view(
                    torch.int8 if int8 else torch.float8_e4m3fn)
                vq = torch.empty_like(kq)
                ks = torch.empty((B, K, S), dtype=torch.float32, device="cuda")
                vs = torch.empty_like(ks)
                c = binding.KVCache(kq, vq, None, k_scale=ks, v_scale=vs)
                binding.gqa_kv_append(c, kt, vt, zero)
                self.caches.append(c)
            del kt, vt
        for i in range(0 if fp8 else n):
            k = k0 if i == 0 else k0.clone()
            v = v0 if i == 0 else v0.clone()
            self.caches.append(binding.KVCache(k, v, bt))
        self.out = torch.empty_like(self.q)
        nbytes = binding.gqa_decode_workspace_bytes(wl.B, wl.H, wl.K, wl.d, self.max_ctx)
        if mq > 1:
            # the mq newest positions of every sequence (already in the cache)
            g = torch.Generator(device="cuda").manual_seed(wl.seed)
            self.qm = torch.randn((wl.B, mq, wl.H, wl.d), generator=g, device="cuda").to(torch.bfloat16)
            self.outm = torch.empty_like(self.qm)
            nbytes = max(nbytes, binding.gqa_decode_multi_workspace_bytes(wl.B, wl.H, wl.K, wl.d, mq, self.max_ctx))
        self.ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        log(f"{wl.name}: {n} cache copies, sum ctx {int(inp.ctx.sum())}, "
            f"{self.alg_bytes / 1e6:.1f} MB per decode, setup {time.time() - t0:.1f}s")

    def append(self, i):
        from grouped_query_attention_gqa_amd import binding
        binding.gqa_kv_append(self.caches[i % len(self.caches)], self.k_new, self.v_new, self.start)

    def step(self, i):
        from grouped_query_attention_gqa_amd import binding
        binding.gqa_decode_step(self.q, self.k_new, self.v_new, self.caches[i % len(self.caches)], self.ctx_d,
                                self.max_ctx, out=self.out, scale=self.wl.scale, workspace=self.ws,
                                window=self.wl.window)

    def multi(self, i):
        from grouped_query_attention_gqa_amd import binding
        binding.gqa_decode_multi(self.qm, self.caches[i % len(self.caches)], self.ctx_d, self.max_ctx, out=self.outm,
                                 scale=self.wl.scale, workspace=self.ws, window=self.wl.window)

    def decode(self, i):
        from grouped_query_attention_gqa_amd import binding
        binding.gqa_decode(self.q, self.caches[i % len(self.caches)], self.ctx_d, self.max_ctx, out=self.out,
                           scale=self.wl.scale, workspace=self.ws, window=self.wl.window)


def time_decode_only(db: DecodeBench, iters: int, warmup: int, call=None):
    """Average decode kernel time (ms) from HIP events on the launch stream
    (`call`: DecodeBench.decode by default, or DecodeBench.step)."""
    import torch
    call = db.decode if call is None else call
    # warm-up: at least `warmup` calls and ~0.2 s of work (see bench_prefill)
    t_end = time.perf_counter() + 0.2
    i = 0
    while i < warmup or time.perf_counter() < t_end:
        call(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for i, (a, b) in enumerate(evs):
        a.record()
        call(i)
        b.record()
    torch.cuda.synchronize()
    ts = [a.elapsed_time(b) for a, b in evs]
    return float(np.mean(ts)), float(np.median(ts))


# ---------------------------------------------------------------------------
# traffic figures from the committed rocprofv3 counter summaries
# ---------------------------------------------------------------------------

def source_code_only(text: str) -> str:
    """C/C++ source without its comments, each run of whitespace made one
    space: what the compiler sees, so that an edit of a comment keeps a hash
    of it.  String and character literals are kept as written."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(names=DECODE_SOURCES) -> str:
    """Hash of the code (comments left out) of the kernel sources the traffic
    counters were taken on, and of the compiler flags they are built with."""
    from grouped_query_attention_gqa_amd import build as gbuild
    h = hashlib.sha256()
    for name in names:
        with open(os.path.join(ROOT, "grouped_query_attention_gqa_amd", "csrc", name), encoding="utf-8") as f:
            h.update(source_code_only(f.read()).encode())
        h.update(" ".join(gbuild.COMMON_FLAGS + gbuild.FILE_FLAGS.get(name, [])).encode())
    return h.hexdigest()[:16]


def committed_traffic(key: str):
    """HBM bytes per call from profiles/traffic.json, if they were taken on the
    current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        return None
    ent = table.get(key)
    if not ent or ent.get("source_sha") != kernel_source_hash(tuple(ent.get("sources", ()))):
        return None
    return ent.get("bytes_per_launch")


def record_traffic(key: str, fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str,
                   algorithmic: int):
    """Writes the byte counters of one leg (FETCH_SIZE and WRITE_SIZE runs, each
    scaled by a device copy's reading) into profiles/traffic.json, tagged with
    the hash of the kernel sources, and prints the summary lines."""
    summ = summarize_traffic(fetch_dir, write_dir, copy_fetch_dir, copy_write_dir, COPY_BYTES)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            table = json.load(f)
    except (OSError, ValueError):
        table = {}
    sources = TRAFFIC_SOURCES[key]
    total = sum(k["hbm_bytes"] for k in summ["kernels"].values())
    table[key] = {"source_sha": kernel_source_hash(sources), "sources": list(sources), "bytes_per_launch": total,
                  "algorithmic_bytes": algorithmic, "kernels": summ["kernels"],
                  "calibration": {k: summ[k] for k in ("copy_bytes", "copy_FETCH_SIZE_KiB", "copy_WRITE_SIZE_KiB",
                                                       "fetch_scale", "write_scale")}}
    with open(path, "w") as f:
        json.dump(table, f, indent=1, sort_keys=True)
    print(key)
    for name, k in summ["kernels"].items():
        print(f"  {name[:60]:60s} FETCH {k['FETCH_SIZE_KiB']:12.1f} KiB  WRITE {k['WRITE_SIZE_KiB']:10.1f} KiB  -> "
              f"{k['hbm_bytes']:12d} B")
    if algorithmic:
        print(f"  one call: {total} B measured vs {algorithmic} B algorithmic (ratio {total / algorithmic:.3f})")


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def summarize_trace(d: str):
    """Per-kernel call count and average duration from a rocprofv3 --kernel-trace --stats run."""
    rows = _csv_rows(os.path.join(d, "run_kernel_stats.csv"))
    lines = [f"{'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'total_%':>8}  kernel"]
    for r in rows:
        lines.append(f"{int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:10.2f} "
                     f"{float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):8.2f}  {r['Name'][:110]}")
    return "\n".join(lines)


def counter_means(d: str):
    """Mean value per (kernel, counter) over the dispatches of a rocprofv3 --pmc run."""
    acc = {}
    for r in _csv_rows(os.path.join(d, "run_counter_collection.csv")):
        k = (r["Kernel_Name"], r["Counter_Name"])
        acc.setdefault(k, []).append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def summarize_traffic(fetch_dir: str, write_dir: str, copy_fetch_dir: str, copy_write_dir: str, copy_bytes: int):
    """HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB), each scaled by what the same
    counter reads for a device copy of `copy_bytes` bytes (reads copy_bytes, writes copy_bytes)."""
    def find(means, pat, ctr):
        for (k, c), (v, n) in means.items():
            if pat in k and c == ctr:
                return v, n
        raise KeyError(pat)
    cf = counter_means(copy_fetch_dir)
    cw = counter_means(copy_write_dir)
    f_copy, _ = find(cf, "copyBuffer", "FETCH_SIZE")
    w_copy, _ = find(cw, "copyBuffer", "WRITE_SIZE")
    f_scale = copy_bytes / (f_copy * 1024.0)
    w_scale = copy_bytes / (w_copy * 1024.0)
    kf = counter_means(fetch_dir)
    kw = counter_means(write_dir)
    out = {"copy_bytes": copy_bytes, "copy_FETCH_SIZE_KiB": f_copy, "copy_WRITE_SIZE_KiB": w_copy,
           "fetch_scale": round(f_scale, 4), "write_scale": round(w_scale, 4), "kernels": {}}
    # the call's kernels run once per call; set-up kernels (filling the
    # caches) run a few times only and are left out
    most = max((n for (k, c), (v, n) in kf.items() if c == "FETCH_SIZE"), default=0)
    for (k, c), (v, n) in kf.items():
        if c != "FETCH_SIZE" or "copyBuffer" in k or "at::native" in k or n < most // 2:
            continue
        w = next((vv for (kk, cc), (vv, nn) in kw.items() if kk == k and cc == "WRITE_SIZE"), 0.0)
        out["kernels"][k[:110]] = {"dispatches": n, "FETCH_SIZE_KiB": round(v, 1), "WRITE_SIZE_KiB": round(w, 1),
                                   "hbm_bytes": int(v * 1024 * f_scale + w * 1024 * w_scale)}
    return out


# ---------------------------------------------------------------------------
# CPU baseline: the oracle on the host cores
# ---------------------------------------------------------------------------

def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def _oracle_threads() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_baseline(db: DecodeBench, budget_s: float = 8.0):
    """The oracle (fp64, untuned) over whole decode steps of the headline workload."""
    import oracle
    wl, inp = db.wl, db.inp
    oracle._load()
    q64 = oracle.to_f64(inp.q, wl.dtype)
    seqs = list(range(wl.B))
    prepared = []
    for b in seqs:
        n = int(inp.ctx[b])
        prepared.append((b, n, oracle.to_f64(inp.k[b:b + 1, :, :n], wl.dtype),
                         oracle.to_f64(inp.v[b:b + 1, :, :n], wl.dtype)))
    rows = np.array([[0, 0, h] for h in range(wl.H)], np.int32)
    kn, vn = inp.new_token_rows()
    done_bytes, t_total, passes = 0, 0.0, 0
    while t_total < budget_s and passes < 50:
        t0 = time.perf_counter()
        for b, n, kb, vb in prepared:
            # the oracle's append of the newest token, then its attention rows
            kc = inp.k[b:b + 1].copy()
            oracle.kv_append(kc, kn[b:b + 1], [n - 1])
            oracle.attention_rows(q64[b:b + 1], kb, vb, [n - 1], [n], False, wl.scale, rows)
        t_total += time.perf_counter() - t0
        done_bytes += db.alg_bytes + append_bytes(wl, 1)
        passes += 1
    threads = _oracle_threads()
    return {
        "value": round(done_bytes / t_total / 1e9, 3),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "cpu_model": cpu_model(),
        "sample": f"the whole {wl.name} decode step (all {wl.B} sequences x {wl.H} heads, append + "
                  f"attention, fp64), {passes} pass(es) in {t_total:.1f} s on {threads} threads",
    }


def _time_oracle(fn, budget_s: float, max_passes: int = 1000):
    """Passes of fn() until budget_s of work (at least one); returns (passes, seconds)."""
    t_total, passes = 0.0, 0
    while passes < max_passes and (passes == 0 or t_total < budget_s):
        t0 = time.perf_counter()
        fn()
        t_total += time.perf_counter() - t0
        passes += 1
    return passes, t_total


def cpu_baseline_workloads(budget_s: float = 3.0):
    """The oracle on the other workloads, each on a bounded sample of the same
    shapes and value distributions, scaled to the metric's unit: decode in GB/s
    of algorithmic bytes, prefill in GFLOP/s of causal work, the tiny fp32
    workloads in microseconds per whole call."""
    import oracle
    from grouped_query_attention_gqa_amd import workloads as W
    oracle._load()
    res = {}
    # tiny fp32 prefill and decode: the whole call
    wl = W.WORKLOADS["tiny_prefill_f32"]
    inp = W.make_prefill(wl)
    q = oracle.to_f64(inp.q, "f32")
    k64 = oracle.to_f64(np.ascontiguousarray(inp.k_new.transpose(0, 2, 1, 3)), "f32")
    v64 = oracle.to_f64(np.ascontiguousarray(inp.v_new.transpose(0, 2, 1, 3)), "f32")
    n, t = _time_oracle(lambda: oracle.attention(q, k64, v64, inp.start_pos, inp.start_pos + wl.s, True, wl.scale),
                        0.5)
    res[wl.name] = {"us_per_call": round(t / n * 1e6, 1), "sample": f"the whole call, {n} passes"}
    wl = W.WORKLOADS["tiny_decode_f32"]
    inp = W.make_decode(wl)
    n0 = int(inp.ctx[0])
    q, k64, v64 = (oracle.to_f64(x, "f32") for x in (inp.q, inp.k[:, :, :n0], inp.v[:, :, :n0]))
    n, t = _time_oracle(lambda: oracle.attention(q, k64, v64, inp.ctx - 1, inp.ctx, False, wl.scale), 0.5)
    res[wl.name] = {"us_per_call": round(t / n * 1e6, 1), "sample": f"the whole call, {n} passes"}
    # decode shapes: a few whole sequences (every head) of the same shape
    for name, b_sample in (("llama2_70b_decode", 2), ("paged_long_decode", 6)):
        wl = W.WORKLOADS[name].replace(B=b_sample)
        inp = W.make_decode(wl, fill="zero")
        q64 = oracle.to_f64(inp.q, wl.dtype)
        rows = np.array([[0, 0, h] for h in range(wl.H)], np.int32)
        # as in the headline leg, the rows are decoded to fp64 (and paged
        # sequences gathered through their table) before the timed passes
        prepared = []
        for b in range(wl.B):
            n_b = int(inp.ctx[b])
            if inp.block_table is None:
                kb, vb = inp.k[b:b + 1, :, :n_b], inp.v[b:b + 1, :, :n_b]
            else:
                kb = oracle.gather_paged_raw(inp.k, inp.block_table[b:b + 1], inp.ctx[b:b + 1], n_b, 0)
                vb = oracle.gather_paged_raw(inp.v, inp.block_table[b:b + 1], inp.ctx[b:b + 1], n_b, 0)
            prepared.append((b, n_b, oracle.to_f64(kb, wl.dtype), oracle.to_f64(vb, wl.dtype)))

        def one_pass():
            for b, n_b, kb, vb in prepared:
                oracle.attention_rows(q64[b:b + 1], kb, vb, [n_b - 1], [n_b], False, wl.scale, rows)
        n, t = _time_oracle(one_pass, budget_s)
        nbytes = decode_bytes(wl, inp.ctx)
        res[name] = {"GB/s": round(nbytes * n / t / 1e9, 3),
                     "sample": f"{b_sample} whole sequences of the {name} shape (ctx {[int(c) for c in inp.ctx]}, "
                               f"every head, fp64), {n} pass(es) in "
                               f"{t:.1f} s"}
    # causal prefill: randomly chosen (sequence, position, head) rows of the
    # full workload, each against its whole causal key range
    wl = W.WORKLOADS["causal_prefill_4k"]
    inp = W.make_prefill(wl)
    rng = np.random.default_rng(7)
    n_rows = 512
    rows = np.stack([rng.integers(0, wl.B, n_rows), rng.integers(0, wl.s, n_rows), rng.integers(0, wl.H, n_rows)],
                    axis=1).astype(np.int32)
    q64 = oracle.to_f64(inp.q, wl.dtype)
    k64 = oracle.to_f64(np.ascontiguousarray(inp.k_new.transpose(0, 2, 1, 3)), wl.dtype)
    v64 = oracle.to_f64(np.ascontiguousarray(inp.v_new.transpose(0, 2, 1, 3)), wl.dtype)
    flops = 4 * wl.d * int(np.sum(rows[:, 1].astype(np.int64) + 1))
    n, t = _time_oracle(lambda: oracle.attention_rows(q64, k64, v64, inp.start_pos, inp.start_pos + wl.s, True,
                                                      wl.scale, rows), budget_s)
    gfs = flops * n / t / 1e9
    res[wl.name] = {"GFLOP/s": round(gfs, 3),
                    "full_call_s_estimate": round(causal_flops(wl) / (gfs * 1e9), 1),
                    "sample": f"{n_rows} random (sequence, position, head) rows of the full workload, each over its "
                              f"whole causal key range ({flops / 1e9:.2f} GFLOP), {n} pass(es) in {t:.1f} s"}
    return res


def pages_context():
    """The pages' own figures, with their hardware: context for the numbers
    above, not targets.  The first one is recomputed with the library's
    cache-size call."""
    from grouped_query_attention_gqa_amd import binding
    layers, tokens = 80, 2048
    mha = binding.gqa_cache_elems_per_token(64, 128) * tokens * layers
    gqa = binding.gqa_cache_elems_per_token(8, 128) * tokens * layers
    return [
        {"figure": f"Llama-2-70B KV cache for 2048 tokens over 80 layers: {mha:,} elements with 64 KV heads (MHA) "
                   f"against {gqa:,} with 8 (GQA), which the page writes as about 2.68 and 0.33 'GB'",
         "source": "concept page (compassingai.com), 关键参数 #2", "hardware": "none (arithmetic)",
         "recomputed": {"mha_elements": mha, "gqa_elements": gqa, "ratio": mha / gqa}},
        {"figure": "GQA instead of MHA raises serving throughput by about 30-50% (a 70B model, 8k context, large "
                   "batches), a figure the page credits to an NVIDIA blog",
         "source": "concept page (compassingai.com), 关键参数 #4", "hardware": "NVIDIA H100"},
        {"figure": "a 7B model (Qwen2-7B with Int4 weights and an fp16 KV cache) served on a single 40 GB A100",
         "source": "blog post (discosf.com), §1", "hardware": "NVIDIA A100 40G"},
    ]


def bench_tiny(iters: int, warmup: int):
    """The tiny fp32 workloads (causal prefill of s = 128; decode over 128
    cached tokens): launch-bound, reported in microseconds per call.  `us` is
    the device time per call, from a HIP graph of 20 calls replayed back to
    back (no host work between the calls); `eager_us` brackets single eager
    calls with HIP events, so it also holds the host's launch path."""
    import torch
    from grouped_query_attention_gqa_amd import binding
    from grouped_query_attention_gqa_amd import workloads as W
    out = {}
    wl = W.WORKLOADS["tiny_prefill_f32"]
    inp = W.make_prefill(wl)
    q, kn, vn, start = up(inp.q), up(inp.k_new), up(inp.v_new), up(inp.start_pos)
    kc = torch.zeros(wl.B, wl.K, wl.s, wl.d, dtype=torch.float32, device="cuda")
    cache = binding.KVCache(kc, torch.zeros_like(kc))
    o = torch.empty_like(q)
    out[wl.name] = _tiny_times(lambda: binding.gqa_prefill(q, kn, vn, cache, start, causal=True, out=o,
                                                           scale=wl.scale), iters, warmup)
    wl = W.WORKLOADS["tiny_decode_f32"]
    db = DecodeBench(wl, copies=1)
    out[wl.name] = _tiny_times(lambda: db.decode(0), iters, warmup)
    return out


def _tiny_times(call, iters, warmup, per_graph=20):
    import torch
    for _ in range(warmup):
        call()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    eager = np.array([a.elapsed_time(b) for a, b in evs])
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(per_graph):
            call()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(3, iters // per_graph)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    dev_us = a.elapsed_time(b) * 1e3 / (reps * per_graph)
    del g
    return {"us": round(dev_us, 2), "eager_us": round(float(np.mean(eager)) * 1e3, 2),
            "eager_median_us": round(float(np.median(eager)) * 1e3, 2), "calls": reps * per_graph}


# ---------------------------------------------------------------------------

def main():
    args = parse()
    if args.summarize:
        print(summarize_trace(args.summarize))
        return
    if args.traffic:
        key, fd, wd, cfd, cwd, alg = args.traffic
        record_traffic(key, fd, wd, cfd, cwd, int(alg))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU; --gpus above 1 is not supported",
                          "n_gpus": args.gpus}))
        sys.stderr.write("bench.py: only --gpus 1 is supported: the library runs on one GPU\n")
        sys.exit(2)
    import torch
    from grouped_query_attention_gqa_amd import binding
    from grouped_query_attention_gqa_amd import workloads as W
    if not torch.cuda.is_available():
        sys.stderr.write("bench.py needs a GPU\n")
        sys.exit(1)
    binding.load_library()
    torch.cuda.set_device(0)

    if args.only:
        return profile_only(args)

    # ---- headline: Llama-3-8B-shaped decode step ---------------------------
    wl = W.WORKLOADS["llama3_8b_decode"]
    db = DecodeBench(wl)
    step_bytes = db.alg_bytes + append_bytes(wl, 1)
    # warm-up: at least `warmup` steps and ~0.2 s of work (see bench_prefill)
    t_end = time.perf_counter() + 0.2
    i = 0
    while i < args.warmup or time.perf_counter() < t_end:
        db.step(i)
        i += 1
        if i % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # the timed steps: wall clock over exactly `steps` calls
    t0 = time.perf_counter()
    for i in range(args.steps):
        db.step(i)
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    # the kernels' own time: HIP events around each call on its stream
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record()
        db.step(i)
        ev[i][1].record()
    torch.cuda.synchronize()
    ev_ms = np.array([a.elapsed_time(b) for a, b in ev])
    dec_ms = float(np.mean(ev_ms))
    value = step_bytes / (ms_step * 1e-3) / 1e9
    achieved = step_bytes / (dec_ms * 1e-3) / 1e9
    traffic = committed_traffic("decode/llama3_8b_decode")
    log(f"decode step {ms_step * 1e3:.1f} us ({value:.0f} GB/s); step kernels {dec_ms * 1e3:.1f} us "
        f"({achieved:.0f} GB/s, {100 * achieved / HBM_PEAK_GBS:.1f}% of peak)")
    # the same step as two calls (append, then decode), timed the same way
    t0 = time.perf_counter()
    for i in range(args.steps):
        db.append(i)
        db.decode(i)
    torch.cuda.synchronize()
    two_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    log(f"two-call step (append, then decode) {two_ms * 1e3:.1f} us")

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "K": wl.K, "d": wl.d,
                   "ctx": "U[1024,4096] per sequence", "sum_ctx": int(db.ctx.sum()),
                   "step": "gqa_decode_step (append of the newest token + decode, one call)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "kernel": DECODE_KERNELS,
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "bytes_per_launch": step_bytes, "avg_launch_us": round(dec_ms * 1e3, 2),
                     "median_launch_us": round(float(np.median(ev_ms)) * 1e3, 2),
                     "p90_launch_us": round(float(np.percentile(ev_ms, 90)) * 1e3, 2)},
        "two_call_step": {"us": round(two_ms * 1e3, 2), "GB/s": round(step_bytes / (two_ms * 1e-3) / 1e9, 1),
                          "calls": "gqa_kv_append + gqa_decode"},
    }
    del db
    torch.cuda.empty_cache()
    # context: what the device streams from HBM with nothing else running
    sus = sustained_hbm_read()
    if sus:
        best = max(sus.values())
        result["roofline"]["sustained_hbm_read_gbs"] = sus
        result["roofline"]["frac_of_sustained"] = round(achieved / best, 4)
        log(f"sustained HBM read: {best:.0f} GB/s; the step's kernels reach {100 * achieved / best:.1f}%")

    if not args.no_extra:
        # ---- causal prefill ------------------------------------------------
        result["prefill"] = bench_prefill(W.WORKLOADS["causal_prefill_4k"], max(LEG_CALLS, args.steps), 5, probe=True)
        torch.cuda.empty_cache()
        # ---- the other decode shapes --------------------------------------
        extra = {}
        for name in ("llama2_70b_decode", "paged_long_decode", "llama2_70b_decode_mha", "llama2_70b_decode_mqa",
                     "mistral_7b_window_decode", "d64_decode"):
            w = W.WORKLOADS[name]
            d2 = DecodeBench(w)
            mean_ms, med_ms = time_decode_only(d2, max(LEG_CALLS, args.steps), 3)
            gbs = d2.alg_bytes / (mean_ms * 1e-3) / 1e9
            extra[name] = {"us": round(mean_ms * 1e3, 2), "GB/s": round(gbs, 1),
                           "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4), "bytes": d2.alg_bytes,
                           "median_us": round(med_ms * 1e3, 2), "calls": max(LEG_CALLS, args.steps),
                           "traffic": committed_traffic("decode/" + name)}
            log(f"{name}: {mean_ms * 1e3:.1f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)")
            del d2
            torch.cuda.empty_cache()
        # ---- four newest positions per sequence at once (speculative verify) -
        w = W.WORKLOADS["llama3_8b_decode"]
        d2 = DecodeBench(w, mq=4)
        mean_ms, med_ms = time_decode_only(d2, max(LEG_CALLS, args.steps), 3, d2.multi)
        gbs = d2.alg_bytes / (mean_ms * 1e-3) / 1e9
        extra["llama3_8b_decode_4_positions"] = {
            "us": round(mean_ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": d2.alg_bytes, "call": "gqa_decode_multi, s = 4 causal positions per sequence"}
        log(f"llama3_8b_decode_4_positions: {mean_ms * 1e3:.1f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)")
        del d2
        torch.cuda.empty_cache()
        # ---- the Llama-3-8B decode on an FP8 (E4M3, scale per row) cache ----
        w = W.WORKLOADS["llama3_8b_decode"]
        d2 = DecodeBench(w, fp8=True)
        mean_ms, med_ms = time_decode_only(d2, max(LEG_CALLS, args.steps), 3)
        gbs = d2.alg_bytes / (mean_ms * 1e-3) / 1e9
        extra["llama3_8b_decode_fp8_cache"] = {
            "us": round(mean_ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": d2.alg_bytes, "cache": "FP8 E4M3 codes + one fp32 scale per row; q/out bf16",
            "median_us": round(med_ms * 1e3, 2), "calls": max(LEG_CALLS, args.steps),
            "traffic": committed_traffic("decode/llama3_8b_decode_fp8_cache")}
        log(f"llama3_8b_decode_fp8_cache: {mean_ms * 1e3:.1f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)")
        del d2
        torch.cuda.empty_cache()
        # ---- the same on an INT8 (scale per row) cache ----------------------
        d2 = DecodeBench(w, int8=True)
        mean_ms, med_ms = time_decode_only(d2, max(LEG_CALLS, args.steps), 3)
        gbs = d2.alg_bytes / (mean_ms * 1e-3) / 1e9
        extra["llama3_8b_decode_int8_cache"] = {
            "us": round(mean_ms * 1e3, 2), "GB/s": round(gbs, 1), "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
            "bytes": d2.alg_bytes, "cache": "INT8 codes + one fp32 scale per row; q/out bf16",
            "median_us": round(med_ms * 1e3, 2), "calls": max(LEG_CALLS, args.steps),
            "traffic": committed_traffic("decode/llama3_8b_decode_int8_cache")}
        log(f"llama3_8b_decode_int8_cache: {mean_ms * 1e3:.1f} us, {gbs:.0f} GB/s ({100 * gbs / HBM_PEAK_GBS:.1f}%)")
        del d2
        torch.cuda.empty_cache()
        result["decode_workloads"] = extra
        # ---- chunked prefill: new tokens after a cached prefix, paged ----
        result["prefill_workloads"] = {
            "chunked_prefill_paged": bench_prefill(W.WORKLOADS["chunked_prefill_paged"], max(LEG_CALLS, args.steps), 5),
            "chunked_prefill_paged_fp8_cache": bench_prefill(W.WORKLOADS["chunked_prefill_paged"],
                                                             max(LEG_CALLS, args.steps), 5, fp8=True),
            "chunked_prefill_paged_int8_cache": bench_prefill(W.WORKLOADS["chunked_prefill_paged"],
                                                              max(LEG_CALLS, args.steps), 5, int8=True)}
        torch.cuda.empty_cache()

        # ---- the tiny fp32 workloads: launch-bound, in microseconds --------
        result["tiny_workloads"] = bench_tiny(max(LEG_CALLS, args.steps), 10)
        log(f"tiny workloads: {result['tiny_workloads']}")

    if not args.no_cpu_baseline:
        wl = W.WORKLOADS["llama3_8b_decode"]
        db = DecodeBench(wl, copies=1)
        result["cpu_baseline"] = cpu_baseline(db)
        del db
        torch.cuda.empty_cache()
        if not args.no_extra:
            result["cpu_baseline"]["workloads"] = cpu_baseline_workloads()
        log(f"cpu baseline: {result['cpu_baseline']}")
    result["pages_context"] = pages_context()

    print(json.dumps(result), flush=True)


def sustained_hbm_read():
    """The rate (GB/s) at which the device streams a 1 GiB buffer (four times
    the Infinity Cache) into its compute units with nothing else running, from
    the probe library beside libgqa.so: 16-byte loads, eight in flight per
    thread, plain and non-temporal, with four and eight workgroups of 256
    threads per CU; HIP events on the current stream.  Returns the rates by
    configuration, or None when the probe library is missing."""
    import ctypes
    import torch
    from grouped_query_attention_gqa_amd import build as gbuild
    if not os.path.exists(gbuild.PROBE_LIB):
        return None
    lib = ctypes.CDLL(gbuild.PROBE_LIB)
    lib.gqa_probe_stream_read.restype = ctypes.c_int
    lib.gqa_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    nbytes = 1 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.empty(cus * 8 * 256, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    reps, out = 20, {}
    for nt in (0, 1):
        for per_cu in (4, 8):
            wgs = cus * per_cu
            def call():
                rc = lib.gqa_probe_stream_read(buf.data_ptr(), nbytes, sink.data_ptr(), sink.numel(), wgs, nt, stream)
                if rc != 0:
                    raise RuntimeError(f"gqa_probe_stream_read failed ({rc})")
            t_end = time.perf_counter() + 0.2
            while time.perf_counter() < t_end:
                for _ in range(8):
                    call()
                torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                call()
            b.record()
            torch.cuda.synchronize()
            label = ("nontemporal" if nt else "plain") + f"_{per_cu}_wg_per_cu"
            out[label] = round(nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
    del buf
    torch.cuda.empty_cache()
    return out


def sustained_mfma(operands):
    """The rate (TFLOP/s) at which the device sustains v_mfma_f32_32x32x16_bf16
    with nothing else running, from the probe library beside libgqa.so: with
    `operands` (a device tensor whose bytes are read as bf16 values; the
    prefill leg passes its own q), and with all-zero operands.  One wave per
    SIMD, each with four independent accumulators; HIP events on the current
    stream."""
    import ctypes
    import torch
    from grouped_query_attention_gqa_amd import build as gbuild
    if not os.path.exists(gbuild.PROBE_LIB):
        return None
    lib = ctypes.CDLL(gbuild.PROBE_LIB)
    lib.gqa_probe_mfma_rate.restype = ctypes.c_int
    lib.gqa_probe_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    lib.gqa_probe_mfma_count.restype = ctypes.c_int64
    lib.gqa_probe_mfma_count.argtypes = [ctypes.c_int, ctypes.c_int]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    sink = torch.empty(cus * 512, dtype=torch.float32, device="cuda")
    zeros = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    iters, reps = 2000, 20
    out = {}
    for label, buf in (("workload_operands", operands), ("zero_operands", zeros)):
        for w in (1,):
            def call():
                rc = lib.gqa_probe_mfma_rate(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                                             sink.numel(), w, iters, stream)
                if rc != 0:
                    raise RuntimeError(f"gqa_probe_mfma_rate failed ({rc})")
            # ~0.3 s of the same work first, as for the timed legs: the clock
            # under matrix load settles over milliseconds
            t_end = time.perf_counter() + 0.3
            while time.perf_counter() < t_end:
                for _ in range(8):
                    call()
                torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                call()
            b.record()
            torch.cuda.synchronize()
            flop = 32768.0 * lib.gqa_probe_mfma_count(w, iters) * reps
            out[f"{label}_{w}_wave_per_simd"] = round(flop / (a.elapsed_time(b) * 1e-3) / 1e12, 1)
    return out


def bench_prefill(wl, iters, warmup, fp8=False, probe=False, int8=False):
    """Append + attention of the prefill workload, HIP events per call.  fp8:
    the cache holds E4M3 codes and a scale per row (the new rows are quantised
    by the call)."""
    import torch
    from grouped_query_attention_gqa_amd import binding
    from grouped_query_attention_gqa_amd import workloads as W
    inp = W.make_prefill(wl)
    q, kn, vn, start = up(inp.q), up(inp.k_new), up(inp.v_new), up(inp.start_pos)
    S = wl.start + wl.s
    if wl.paged:
        # a shuffled block table over a pool just large enough; the cached
        # prefix holds zeros (its values do not change the work)
        rng = np.random.default_rng(wl.seed)
        table, n_pool = W.deal_blocks(rng, np.full(wl.B, S, np.int32), wl.block_size)
        shape = (n_pool, wl.K, wl.block_size, wl.d)
    else:
        table, shape = None, (wl.B, wl.K, S, wl.d)
    quant = "int8" if int8 else "fp8" if fp8 else None
    if quant:
        kc = torch.zeros(shape, dtype=torch.uint8, device="cuda").view(torch.int8 if int8 else torch.float8_e4m3fn)
        vc = torch.zeros_like(kc)
        ks = torch.zeros(shape[:3], dtype=torch.float32, device="cuda")
        cache = binding.KVCache(kc, vc, None if table is None else up(table), k_scale=ks, v_scale=torch.zeros_like(ks))
    else:
        kc = torch.zeros(shape, dtype=torch.bfloat16, device="cuda")
        cache = binding.KVCache(kc, torch.zeros_like(kc), None if table is None else up(table))
    out = torch.empty_like(q)
    # warm-up: at least `warmup` calls and ~0.3 s of work, so that the
    # clocks have left the idle state the host-side input generation leaves
    t_end = time.perf_counter() + 0.3
    n = 0
    while n < warmup or time.perf_counter() < t_end:
        binding.gqa_prefill(q, kn, vn, cache, start, causal=True, out=out, scale=wl.scale, window=wl.window)
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record()
        binding.gqa_prefill(q, kn, vn, cache, start, causal=True, out=out, scale=wl.scale, window=wl.window)
        b.record()
    torch.cuda.synchronize()
    ev_ms = np.array([a.elapsed_time(b) for a, b in evs])
    ms = float(np.mean(ev_ms))
    flops = causal_flops(wl)
    tf = flops / (ms * 1e-3) / 1e12
    log(f"prefill {wl.name}: {ms * 1e3:.1f} us (append + attention), {tf:.1f} TFLOP/s "
        f"({100 * tf / BF16_MFMA_PEAK_TFLOPS:.1f}% of bf16 MFMA peak)")
    roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": BF16_MFMA_PEAK_TFLOPS,
            "unit": "TFLOP/s", "frac": round(tf / BF16_MFMA_PEAK_TFLOPS, 4),
            "note": "time covers the append and the attention kernel"}
    if probe:
        # context: what the matrix cores sustain on these operands with no
        # softmax, LDS or memory work (their clock under load depends on the data)
        sus = sustained_mfma(q)
        if sus:
            best = sus["workload_operands_1_wave_per_simd"]
            roof["sustained_mfma_tflops"] = sus
            roof["frac_of_sustained"] = round(tf / best, 4)
            log(f"sustained matrix rate on the leg's q values: {best:.0f} TFLOP/s; the call reaches {100 * tf / best:.1f}%")
    return {"workload": wl.name, "B": wl.B, "s": wl.s, "start": wl.start, "H": wl.H, "K": wl.K, "d": wl.d,
            "paged": wl.paged,
            "cache": {"fp8": "FP8 E4M3 codes + one fp32 scale per row", "int8": "INT8 codes + one fp32 scale per row",
                      None: "bf16"}[quant],
            "us_per_call": round(ms * 1e3, 2),
            "median_us": round(float(np.median(ev_ms)) * 1e3, 2), "p90_us": round(float(np.percentile(ev_ms, 90)) * 1e3, 2),
            "flops": flops, "TFLOP/s": round(tf, 2), "calls": iters,
            "traffic": committed_traffic(("prefill/" + wl.name) + (f"_{quant}_cache" if quant else "")),
            "roofline": roof}


def profile_only(args):
    """A short run of one kernel, for rocprofv3 (no JSON contract)."""
    import torch
    from grouped_query_attention_gqa_amd import workloads as W
    if args.only in ("prefill", "chunked", "chunked_fp8", "chunked_int8"):
        name = "causal_prefill_4k" if args.only == "prefill" else "chunked_prefill_paged"
        r = bench_prefill(W.WORKLOADS[name], args.steps, args.warmup, fp8=args.only == "chunked_fp8",
                          int8=args.only == "chunked_int8")
        print(json.dumps(r), flush=True)
        return
    if args.only in ("tiny_prefill", "tiny_decode"):
        r = bench_tiny(args.steps, args.warmup)
        print(json.dumps(r), flush=True)
        return
    if args.only == "copy":
        # the calibration copy for the byte counters: reads and writes COPY_BYTES per dispatch
        a = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(args.steps):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": COPY_BYTES, "copies": args.steps}), flush=True)
        return
    name = {"decode": "llama3_8b_decode", "step": "llama3_8b_decode", "decode70b": "llama2_70b_decode",
            "paged": "paged_long_decode", "mha": "llama2_70b_decode_mha", "mqa": "llama2_70b_decode_mqa",
            "window": "mistral_7b_window_decode", "fp8": "llama3_8b_decode", "int8": "llama3_8b_decode",
            "multi": "llama3_8b_decode",
            "d64": "d64_decode"}[args.only]
    db = DecodeBench(W.WORKLOADS[name], fp8=args.only == "fp8", mq=4 if args.only == "multi" else 1,
                     int8=args.only == "int8")
    call = {"step": db.step, "multi": getattr(db, "multi", None)}.get(args.only)
    mean_ms, med_ms = time_decode_only(db, args.steps, args.warmup, call)
    print(json.dumps({"workload": name, "decode_us": round(mean_ms * 1e3, 2),
                      "GB/s": round(db.alg_bytes / (mean_ms * 1e-3) / 1e9, 1), "bytes": db.alg_bytes}), flush=True)


if __name__ == "__main__":
    main()
