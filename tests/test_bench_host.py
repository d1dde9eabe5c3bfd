"""Host-side logic of bench.py (no GPU): the one-GPU contract, the
algorithmic byte counts the decode legs are divided by, and the scaling of
the rocprofv3 byte counters by a device copy of known size."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from grouped_query_attention_gqa_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_decode_bytes_count_each_visible_row_once():
    wl = W.WORKLOADS["llama3_8b_decode"]
    ctx = np.array([1024, 4096, 7], np.int32)
    wl3 = wl.replace(B=3)
    # a cached token is one K row and one V row per KV head: 2 * K * d bf16
    # values; q is read and out written once per head
    kv = 2 * wl.K * wl.d * 2 * int(ctx.sum())
    qo = 2 * 3 * wl.H * wl.d * 2
    assert bench.decode_bytes(wl3, ctx) == kv + qo
    # a quantised row is d one-byte codes and one 4-byte scale
    assert bench.decode_bytes(wl3, ctx, fp8=True) == 2 * wl.K * (wl.d + 4) * int(ctx.sum()) + qo
    # with a sliding window only the window's rows count
    ww = wl3.replace(window=100)
    assert bench.decode_bytes(ww, ctx) == 2 * wl.K * wl.d * 2 * (100 + 100 + 7) + qo


def _counter_csv(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_is_scaled_by_the_copy_reading(tmp_path):
    """FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are scaled by the factor
    that turns the same counter's reading of a known copy into its bytes;
    set-up kernels that ran only a few times are left out."""
    cb = bench.COPY_BYTES
    d = {n: str(tmp_path / n) for n in ("cf", "cw", "kf", "kw")}
    _counter_csv(d["cf"], [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "FETCH_SIZE",
                            "Counter_Value": cb / 1024 / 2}])            # the counter reads half the bytes
    _counter_csv(d["cw"], [{"Kernel_Name": "__amd_rocclr_copyBuffer", "Counter_Name": "WRITE_SIZE",
                            "Counter_Value": cb / 1024}])
    main = [{"Kernel_Name": "main_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000.0}] * 10
    setup = [{"Kernel_Name": "fill_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": 9e6}]
    _counter_csv(d["kf"], main + setup)
    _counter_csv(d["kw"], [{"Kernel_Name": "main_kernel", "Counter_Name": "WRITE_SIZE", "Counter_Value": 10.0}] * 10)
    s = bench.summarize_traffic(d["kf"], d["kw"], d["cf"], d["cw"], cb)
    assert s["fetch_scale"] == pytest.approx(2.0) and s["write_scale"] == pytest.approx(1.0)
    assert list(s["kernels"]) == ["main_kernel"]
    assert s["kernels"]["main_kernel"]["hbm_bytes"] == int(1000 * 1024 * 2 + 10 * 1024)


def test_source_hash_ignores_comments_but_not_code():
    src = ('// header\nint f(int x) { /* a block\n comment */ return x + 1; }  // tail\n'
           'const char *s = "// kept: inside a string";\n')
    base = bench.source_code_only(src)
    assert "header" not in base and "block" not in base and "tail" not in base
    assert '"// kept: inside a string"' in base
    # an edited comment or reflowed whitespace: the same code
    assert bench.source_code_only(src.replace("a block", "another").replace("  //", "\n//")) == base
    # an edited statement or string: different code
    assert bench.source_code_only(src.replace("x + 1", "x + 2")) != base
    assert bench.source_code_only(src.replace("kept", "kept!")) != base


def test_committed_traffic_is_keyed_to_the_current_code():
    # every stored byte-counter figure was taken on the kernels as they stand
    for key in bench.TRAFFIC_SOURCES:
        assert bench.committed_traffic(key) is not None, key
