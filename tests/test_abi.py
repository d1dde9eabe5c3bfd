"""The C ABI without a GPU: the library loads, exports what include/gqa.h
declares, and rejects bad arguments before anything reaches the device."""
import ctypes
import os
import re

import pytest

from grouped_query_attention_gqa_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gqa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*[A-Za-z_][\w\s\*]*?\b(gqa_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def lib():
    return binding.load_library()


def test_header_declares_the_three_calls():
    names = declared_functions()
    for n in ("gqa_kv_append", "gqa_decode", "gqa_prefill", "gqa_decode_workspace_bytes",
              "gqa_cache_elems_per_token"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(binding.EXPORTED_SYMBOLS)


def test_abi_version_and_status_strings(lib):
    assert lib.gqa_abi_version() == 3
    assert lib.gqa_status_string(0) == b"ok"
    assert b"workspace" in lib.gqa_status_string(3)


@pytest.mark.parametrize("K,d,expect", [(8, 128, 2048), (64, 128, 16384), (1, 128, 256), (2, 64, 256),
                                        (0, 128, -1), (8, 0, -1)])
def test_cache_elems_per_token(lib, K, d, expect):
    # 2*K*d elements per token per layer (concept page, key parameters #2)
    assert binding.gqa_cache_elems_per_token(K, d) == expect


def test_workspace_plan(lib):
    # tile prefix of one launch (513 int32) + two partial slots per workgroup (512)
    align = lambda x: (x + 255) // 256 * 256
    for (B, H, K, d) in [(16, 64, 8, 128), (1, 8, 2, 64), (64, 64, 1, 128)]:
        G = H // K
        n = binding.gqa_decode_workspace_bytes(B, H, K, d, 8192)
        assert n == align(513 * 4) + align(512 * 2 * G * d * 4) + align(512 * 2 * G * 2 * 4)
    assert binding.gqa_decode_workspace_bytes(1, 8, 3, 64, 128) == 0   # H % K != 0 -> 0
    assert binding.gqa_decode_workspace_bytes(0, 8, 2, 64, 128) == 0


def _cache(**kw):
    s = binding._CacheStruct()
    s.k, s.v = 0x10000, 0x20000          # never dereferenced: every case fails validation
    s.block_table = None
    s.S_max, s.num_kv_heads, s.head_dim, s.dtype = 128, 2, 64, binding.GQA_F32
    s.max_blocks_per_seq, s.block_size, s.num_blocks = 0, 16, 0
    for k, v in kw.items():
        setattr(s, k, v)
    return s


FAKE = ctypes.c_void_p(0x30000)


def _decode(lib, cache, B=1, H=8, max_ctx=128, scale=0.125, ws=None, ws_bytes=0):
    return lib.gqa_decode(FAKE, ctypes.byref(cache), FAKE, max_ctx, B, H, ctypes.c_float(scale), FAKE,
                          ws, ws_bytes, None)


@pytest.mark.parametrize("case,expect", [
    (dict(num_kv_heads=3), binding.GQA_ERR_INVALID_ARG),     # 8 % 3 != 0
    (dict(num_kv_heads=0), binding.GQA_ERR_INVALID_ARG),
    (dict(head_dim=96), binding.GQA_ERR_UNSUPPORTED),
    (dict(head_dim=-1), binding.GQA_ERR_INVALID_ARG),
    (dict(dtype=7), binding.GQA_ERR_UNSUPPORTED),
    (dict(S_max=0), binding.GQA_ERR_INVALID_ARG),
    (dict(k=None), binding.GQA_ERR_INVALID_ARG),
    (dict(block_table=0x40000, block_size=12, max_blocks_per_seq=4, num_blocks=4), binding.GQA_ERR_INVALID_ARG),
    (dict(block_table=0x40000, block_size=16, max_blocks_per_seq=0, num_blocks=4), binding.GQA_ERR_INVALID_ARG),
])
def test_decode_rejects_bad_cache(lib, case, expect):
    assert _decode(lib, _cache(**case)) == expect


def test_decode_rejects_bad_sizes(lib):
    c = _cache()
    assert _decode(lib, c, H=0) == binding.GQA_ERR_INVALID_ARG
    assert _decode(lib, c, B=-1) == binding.GQA_ERR_INVALID_ARG
    assert _decode(lib, c, max_ctx=0) == binding.GQA_ERR_INVALID_ARG
    assert _decode(lib, c, scale=float("nan")) == binding.GQA_ERR_INVALID_ARG
    assert _decode(lib, _cache(num_kv_heads=1), H=128) == binding.GQA_ERR_UNSUPPORTED   # G = 128 > 64
    assert lib.gqa_decode(None, ctypes.byref(c), FAKE, 128, 1, 8, ctypes.c_float(1.0), FAKE, None, 0,
                          None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_decode(FAKE, None, FAKE, 128, 1, 8, ctypes.c_float(1.0), FAKE, None, 0,
                          None) == binding.GQA_ERR_INVALID_ARG
    assert _decode(lib, c, B=0) == binding.GQA_OK                         # empty batch: nothing to do


def test_decode_rejects_small_workspace(lib):
    c = _cache(S_max=8192, num_kv_heads=8, head_dim=128, dtype=binding.GQA_BF16)
    need = lib.gqa_decode_workspace_bytes(16, 64, 8, 128, 8192)
    assert need > 0
    assert _decode(lib, c, B=16, H=64, max_ctx=8192) == binding.GQA_ERR_WORKSPACE
    assert _decode(lib, c, B=16, H=64, max_ctx=8192, ws=FAKE, ws_bytes=need - 1) == binding.GQA_ERR_WORKSPACE


def test_append_and_prefill_reject_bad_args(lib):
    c = _cache()
    assert lib.gqa_kv_append(ctypes.byref(c), None, FAKE, FAKE, 1, 1, None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_kv_append(ctypes.byref(c), FAKE, FAKE, FAKE, -1, 1, None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_kv_append(ctypes.byref(c), FAKE, FAKE, FAKE, 1, 0, None) == binding.GQA_OK
    assert lib.gqa_kv_append(ctypes.byref(_cache(head_dim=80)), FAKE, FAKE, FAKE, 1, 1,
                             None) == binding.GQA_ERR_UNSUPPORTED
    pf = lambda cache, H=8, s=4, scale=0.125: lib.gqa_prefill(FAKE, FAKE, FAKE, ctypes.byref(cache), FAKE, 1, s,
                                                              H, ctypes.c_float(scale), 1, FAKE, None)
    assert pf(_cache(), H=7) == binding.GQA_ERR_INVALID_ARG
    assert pf(_cache(), s=-2) == binding.GQA_ERR_INVALID_ARG
    assert pf(_cache(), scale=float("inf")) == binding.GQA_ERR_INVALID_ARG
    assert pf(_cache(), s=0) == binding.GQA_OK
    assert lib.gqa_prefill(FAKE, FAKE, None, ctypes.byref(_cache()), FAKE, 1, 4, 8, ctypes.c_float(0.1), 1, FAKE,
                           None) == binding.GQA_ERR_INVALID_ARG


def test_decode_step_rejects_bad_args(lib):
    c = _cache()
    step = lambda kn, vn, B=1, H=8: lib.gqa_decode_step(FAKE, kn, vn, ctypes.byref(c), FAKE, 128, B, H,
                                                        ctypes.c_float(0.125), 0, FAKE, None, 0, None)
    assert step(FAKE, None) == binding.GQA_ERR_INVALID_ARG      # both new rows or neither
    assert step(None, FAKE) == binding.GQA_ERR_INVALID_ARG
    assert step(FAKE, FAKE, H=7) == binding.GQA_ERR_INVALID_ARG
    assert step(FAKE, FAKE) == binding.GQA_ERR_WORKSPACE          # checked before any launch
    assert step(FAKE, FAKE, B=0) == binding.GQA_OK


@pytest.mark.parametrize("qdtype", ["fp8", "int8"])
def test_fp8_cache_argument_rules(lib, qdtype):
    """A quantised cache (FP8 E4M3 or INT8) needs both scale arrays and
    head_dim 128; decode takes blocks of at least 16 tokens."""
    f8 = dict(dtype=binding.GQA_FP8_E4M3 if qdtype == "fp8" else binding.GQA_INT8, head_dim=128, S_max=4096,
              num_kv_heads=8)
    sc = dict(k_scale=0x50000, v_scale=0x60000)
    ws = lib.gqa_decode_workspace_bytes(1, 32, 8, 128, 4096)
    dec = lambda cache, H=32: lib.gqa_decode(FAKE, ctypes.byref(cache), FAKE, 4096, 1, H, ctypes.c_float(0.088),
                                             FAKE, FAKE, lib.gqa_decode_workspace_bytes(1, H, 8, 128, 4096), None)
    assert ws > 0
    assert dec(_cache(**f8)) == binding.GQA_ERR_INVALID_ARG                     # no scales
    assert dec(_cache(**f8, k_scale=0x50000)) == binding.GQA_ERR_INVALID_ARG    # one scale array only
    assert dec(_cache(**{**f8, "head_dim": 64}, **sc)) == binding.GQA_ERR_UNSUPPORTED
    paged = dict(block_table=0x40000, block_size=8, max_blocks_per_seq=4, num_blocks=4)
    assert dec(_cache(**f8, **sc, **paged)) == binding.GQA_ERR_UNSUPPORTED      # 8-token blocks
    # prefill over an FP8 cache: head_dim 128 only, both scale arrays
    pf = lambda cache: lib.gqa_prefill(FAKE, FAKE, FAKE, ctypes.byref(cache), FAKE, 1, 4, 32, ctypes.c_float(0.1), 1,
                                       FAKE, None)
    assert pf(_cache(**{**f8, "head_dim": 64}, **sc)) == binding.GQA_ERR_UNSUPPORTED
    assert pf(_cache(**f8, v_scale=0x60000)) == binding.GQA_ERR_INVALID_ARG


def test_unknown_dtype_is_refused(lib):
    assert _decode(lib, _cache(dtype=4)) == binding.GQA_ERR_UNSUPPORTED


@pytest.mark.parametrize("scale", [0.0, -0.125, -0.0, float("-inf")])
def test_every_call_rejects_a_scale_that_is_not_positive(lib, scale):
    """The kernels take each tile's maximum of the raw dot products before
    scaling it, which is the scaled maximum only for a positive scale; zero
    and negative scales are refused before anything is launched."""
    c = _cache()
    sc = ctypes.c_float(scale)
    assert _decode(lib, c, scale=scale) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_decode_window(FAKE, ctypes.byref(c), FAKE, 128, 1, 8, sc, 16, FAKE, FAKE, 1 << 30,
                                 None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_decode_step(FAKE, FAKE, FAKE, ctypes.byref(c), FAKE, 128, 1, 8, sc, 0, FAKE, FAKE, 1 << 30,
                               None) == binding.GQA_ERR_INVALID_ARG
    c128 = _cache(head_dim=128, dtype=binding.GQA_BF16)
    assert lib.gqa_decode_multi(FAKE, ctypes.byref(c128), FAKE, 128, 1, 2, 8, sc, 0, FAKE, FAKE, 1 << 30,
                                None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_prefill(FAKE, FAKE, FAKE, ctypes.byref(c), FAKE, 1, 4, 8, sc, 1, FAKE,
                           None) == binding.GQA_ERR_INVALID_ARG
    assert lib.gqa_prefill_window(FAKE, FAKE, FAKE, ctypes.byref(c), FAKE, 1, 4, 8, sc, 1, 8, FAKE,
                                  None) == binding.GQA_ERR_INVALID_ARG


def test_noalloc_step_checks_arguments_before_touching_the_device(lib):
    """gqa_decode_step_noalloc validates like gqa_decode_step, and refuses a call
    whose workspace exceeds its static buffer, before any HIP call."""
    c = _cache()
    step = lambda kn, vn, B=1, H=8, cache=c, scale=0.125: lib.gqa_decode_step_noalloc(
        FAKE, kn, vn, ctypes.byref(cache), FAKE, 128, B, H, ctypes.c_float(scale), 0, FAKE, None)
    assert step(FAKE, None) == binding.GQA_ERR_INVALID_ARG
    assert step(FAKE, FAKE, H=7) == binding.GQA_ERR_INVALID_ARG
    assert step(FAKE, FAKE, scale=-1.0) == binding.GQA_ERR_INVALID_ARG
    assert step(FAKE, FAKE, B=0) == binding.GQA_OK
    # G = 64 at d = 128: ~33 MiB of partials, beyond the 12 MiB static buffer
    big = _cache(num_kv_heads=1, head_dim=128, dtype=binding.GQA_BF16, S_max=4096)
    assert step(FAKE, FAKE, H=64, cache=big) == binding.GQA_ERR_WORKSPACE


def test_probe_library_stays_outside_the_attention_library(lib):
    # the bench's matrix-rate probe lives in libgqa_probe.so; libgqa.so does not carry it
    from grouped_query_attention_gqa_amd import build as gbuild
    assert not hasattr(lib, "gqa_probe_mfma_rate")
    if not os.path.exists(gbuild.PROBE_LIB):
        pytest.skip("libgqa_probe.so not built")
    probe = ctypes.CDLL(gbuild.PROBE_LIB)
    for name in ("gqa_probe_mfma_rate", "gqa_probe_mfma_count"):
        assert hasattr(probe, name), name
