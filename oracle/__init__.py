"""CPU oracle for grouped-query attention: test infrastructure only.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The library under
``grouped_query_attention_gqa_amd`` never does, and this package imports
nothing from it.

Two independent implementations of the same definition live here:

* ``gqa_oracle.c`` (plain C, fp64, OpenMP over output rows), loaded through
  ctypes by the functions below;
* ``np_oracle.py`` (NumPy fp64, vectorised per KV group), used to cross-check
  the C oracle, plus the streaming (online-softmax, split-and-merge) form the
  pages describe, used to pin that those rewrites are exact.

The definition both follow is the one on the "Grouped-Query Attention"
concept page, section 技术原理, steps 2-4: head h reads KV group
g = h // (H/K), and each row is softmax(q K_g^T / sqrt(d_k)) V_g over the
visible keys.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile gqa_oracle.c into oracle/liboracle.so with gcc (-O2, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        i64, i32, dbl = ctypes.c_int64, ctypes.c_int, ctypes.c_double
        vp = ctypes.c_void_p
        lib.oracle_cache_elems_per_token.restype = i64
        lib.oracle_cache_elems_per_token.argtypes = [i64, i64]
        lib.oracle_kv_cache_elems.restype = i64
        lib.oracle_kv_cache_elems.argtypes = [i64, i64, i64, i64, i64]
        lib.oracle_gqa_attention.restype = i64
        lib.oracle_gqa_attention.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                             vp, vp, i32, dbl, vp]
        lib.oracle_gqa_attention_rows.restype = i64
        lib.oracle_gqa_attention_rows.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                  vp, vp, i32, dbl, i64, vp, vp]
        lib.oracle_gqa_attention_rows_window.restype = i64
        lib.oracle_gqa_attention_rows_window.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32,
                                                         vp, vp, i32, dbl, i32, i64, vp, vp]
        lib.oracle_kv_append.restype = i64
        lib.oracle_kv_append.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32]
        lib.oracle_kv_append_paged.restype = i64
        lib.oracle_kv_append_paged.argtypes = [vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, i32, i32]
        lib.oracle_gather_paged_raw.restype = i64
        lib.oracle_gather_paged_raw.argtypes = [vp, i32, vp, i32, i32, i32, vp, i32, i32, i32, i32, vp]
        lib.oracle_gather_paged.restype = i64
        lib.oracle_gather_paged.argtypes = [vp, vp, i32, i32, i32, vp, i32, i32, i32, i32, vp]
        lib.oracle_e4m3_value.restype = ctypes.c_double
        lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        lib.oracle_e4m3_from_float.restype = ctypes.c_uint8
        lib.oracle_e4m3_from_float.argtypes = [ctypes.c_float]
        lib.oracle_quantize_e4m3_rows.restype = None
        lib.oracle_quantize_e4m3_rows.argtypes = [vp, i64, i32, vp, vp]
        lib.oracle_dequantize_e4m3_rows.restype = None
        lib.oracle_dequantize_e4m3_rows.argtypes = [vp, vp, i64, i32, vp]
        lib.oracle_quantize_i8_rows.restype = None
        lib.oracle_quantize_i8_rows.argtypes = [vp, i64, i32, vp, vp]
        lib.oracle_dequantize_i8_rows.restype = None
        lib.oracle_dequantize_i8_rows.argtypes = [vp, vp, i64, i32, vp]
        _lib = lib
        return lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---------------------------------------------------------------------------
# exact decoding of the stored input formats to fp64
# ---------------------------------------------------------------------------

def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper half of an IEEE binary32; widening is exact."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(x: np.ndarray, dtype: str) -> np.ndarray:
    """Decode stored inputs ('bf16' as uint16 bits, 'f32' as float32) to fp64."""
    if dtype == "bf16":
        return bf16_bits_to_f64(x)
    if dtype == "f32":
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float64)
    if dtype == "f64":
        return np.ascontiguousarray(x, dtype=np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# cache size (concept page 关键参数 #2; inference-optimisation page §6.1)
# ---------------------------------------------------------------------------

def cache_elems_per_token(kv_heads: int, head_dim: int) -> int:
    return int(_load().oracle_cache_elems_per_token(kv_heads, head_dim))


def kv_cache_elems(layers: int, kv_heads: int, head_dim: int, seq_len: int, batch: int) -> int:
    return int(_load().oracle_kv_cache_elems(layers, kv_heads, head_dim, seq_len, batch))


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------

def _i32(a, n):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32).reshape(-1))
    if a.shape[0] != n:
        raise ValueError("per-sequence array has the wrong length")
    return a


def attention(q, k, v, q_start, kv_len, causal: bool, scale: float) -> np.ndarray:
    """All rows.  q [B,Sq,H,d], k/v [B,K,Sk,d] (fp64); returns [B,Sq,H,d] fp64."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Sq, H, d = q.shape
    Bk, K, Sk, dk = k.shape
    if Bk != B or dk != d or v.shape != k.shape:
        raise ValueError("q/k/v shapes disagree")
    qs, kl = _i32(q_start, B), _i32(kv_len, B)
    out = np.empty_like(q)
    rc = _load().oracle_gqa_attention(_ptr(q), _ptr(k), _ptr(v), B, Sq, H, K, d, Sk,
                                      _ptr(qs), _ptr(kl), int(bool(causal)), float(scale), _ptr(out))
    if rc < 0:
        raise ValueError("oracle rejected the shapes")
    return out


def attention_rows(q, k, v, q_start, kv_len, causal: bool, scale: float, rows, window: int = 0) -> np.ndarray:
    """Listed rows only; rows is an int array [n, 3] of (b, i, h); returns [n, d].
    window > 0: each row sees only its `window` most recent positions."""
    q = np.ascontiguousarray(q, dtype=np.float64)
    k = np.ascontiguousarray(k, dtype=np.float64)
    v = np.ascontiguousarray(v, dtype=np.float64)
    B, Sq, H, d = q.shape
    _, K, Sk, _ = k.shape
    rows = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
    qs, kl = _i32(q_start, B), _i32(kv_len, B)
    out = np.empty((rows.shape[0], d), dtype=np.float64)
    rc = _load().oracle_gqa_attention_rows_window(_ptr(q), _ptr(k), _ptr(v), B, Sq, H, K, d, Sk,
                                                  _ptr(qs), _ptr(kl), int(bool(causal)), float(scale), int(window),
                                                  rows.shape[0], _ptr(rows), _ptr(out))
    if rc < 0:
        raise ValueError("oracle rejected the shapes")
    return out


# ---------------------------------------------------------------------------
# cache writes and paged reads
# ---------------------------------------------------------------------------

def kv_append(cache: np.ndarray, new_rows: np.ndarray, start_pos) -> int:
    """In place: cache [B,K,S_max,d] <- new_rows [B,s_new,K,d] at start_pos[b]."""
    if not cache.flags.c_contiguous:
        raise ValueError("cache must be C-contiguous")
    new_rows = np.ascontiguousarray(new_rows)
    if new_rows.dtype != cache.dtype:
        raise ValueError("dtype mismatch")
    B, K, S_max, d = cache.shape
    Bn, s_new, Kn, dn = new_rows.shape
    if (Bn, Kn, dn) != (B, K, d):
        raise ValueError("shape mismatch")
    sp = _i32(start_pos, B)
    return int(_load().oracle_kv_append(_ptr(cache), _ptr(new_rows), _ptr(sp), B, s_new, K, d,
                                        S_max, cache.dtype.itemsize))


def kv_append_paged(pool: np.ndarray, new_rows: np.ndarray, start_pos, block_table) -> int:
    """In place: pool [N,K,bs,d] <- new_rows [B,s_new,K,d] through block_table [B,max_blocks]."""
    if not pool.flags.c_contiguous:
        raise ValueError("pool must be C-contiguous")
    new_rows = np.ascontiguousarray(new_rows)
    N, K, bs, d = pool.shape
    B, s_new, Kn, dn = new_rows.shape
    if (Kn, dn) != (K, d) or new_rows.dtype != pool.dtype:
        raise ValueError("shape/dtype mismatch")
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sp = _i32(start_pos, B)
    return int(_load().oracle_kv_append_paged(_ptr(pool), _ptr(new_rows), _ptr(sp), _ptr(bt),
                                              bt.shape[1], N, bs, B, s_new, K, d,
                                              pool.dtype.itemsize))


def gather_paged(pool_f64: np.ndarray, block_table, ctx_lens, S_out: int) -> np.ndarray:
    """Contiguous [B,K,S_out,d] fp64 copy of a paged pool [N,K,bs,d] (NaN past ctx)."""
    pool_f64 = np.ascontiguousarray(pool_f64, dtype=np.float64)
    N, K, bs, d = pool_f64.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    B = bt.shape[0]
    cl = _i32(ctx_lens, B)
    out = np.empty((B, K, S_out, d), dtype=np.float64)
    bad = _load().oracle_gather_paged(_ptr(pool_f64), _ptr(bt), bt.shape[1], N, bs, _ptr(cl),
                                      B, K, d, S_out, _ptr(out))
    if bad:
        raise ValueError(f"{bad} visible positions map to invalid physical blocks")
    return out


def gather_paged_raw(pool: np.ndarray, block_table, ctx_lens, S_out: int, fill) -> np.ndarray:
    """Contiguous [B,K,S_out,d] copy of a paged pool in its stored format (no decoding);
    positions past each ctx_lens[b] hold ``fill``."""
    pool = np.ascontiguousarray(pool)
    N, K, bs, d = pool.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    B = bt.shape[0]
    cl = _i32(ctx_lens, B)
    out = np.full((B, K, S_out, d), fill, dtype=pool.dtype)
    bad = _load().oracle_gather_paged_raw(_ptr(pool), pool.dtype.itemsize, _ptr(bt), bt.shape[1], N, bs,
                                          _ptr(cl), B, K, d, S_out, _ptr(out))
    if bad:
        raise ValueError(f"{bad} visible positions map to invalid physical blocks")
    return out


def paged_attention_rows(q, pool_k, pool_v, block_table, ctx_lens, scale, rows_per_seq=None,
                         seqs=None, window: int = 0) -> tuple[np.ndarray, np.ndarray]:
    """Decode rows over a paged cache: gather each listed sequence, then attend.

    q is [B,1,H,d] fp64; pool_k/pool_v [N,K,bs,d] fp64.  ``seqs`` lists the
    sequences to evaluate (default all); every head of each is computed.
    Returns (rows [n,3], out [n,d]).
    """
    B, _, H, d = q.shape
    seqs = list(range(B)) if seqs is None else list(seqs)
    bt = np.asarray(block_table, dtype=np.int32)
    cl = np.asarray(ctx_lens, dtype=np.int32)
    outs, rows = [], []
    for b in seqs:
        S = int(cl[b])
        kc = gather_paged(pool_k, bt[b:b + 1], cl[b:b + 1], S)
        vc = gather_paged(pool_v, bt[b:b + 1], cl[b:b + 1], S)
        r = np.array([[0, 0, h] for h in range(H)], dtype=np.int32)
        o = attention_rows(q[b:b + 1], kc, vc, [S - 1], [S], False, scale, r, window)
        outs.append(o)
        rows.append(np.array([[b, 0, h] for h in range(H)], dtype=np.int32))
    return np.concatenate(rows), np.concatenate(outs)


# ---------------------------------------------------------------------------
# FP8 (E4M3) KV cache, one fp32 scale per cached row (inference-optimisation
# page §15.5.1: per-token / per-head scales, FP8 E4M3)
# ---------------------------------------------------------------------------

def e4m3_value(code: int) -> float:
    """The value of one E4M3 code (NaN for the two NaN codes)."""
    return float(_load().oracle_e4m3_value(int(code) & 0xFF))


def e4m3_from_float(x: float) -> int:
    """The E4M3 code nearest to the fp32 value x (ties to even, saturating)."""
    return int(_load().oracle_e4m3_from_float(ctypes.c_float(float(x))))


def quantize_e4m3_rows(x: np.ndarray):
    """Rows x[..., d] (fp32 values; bf16 bits may be given as uint16) -> (codes
    uint8 [..., d], scales float32 [...]): scale = amax / 448 and codes the
    nearest E4M3 values of x / scale, both decided in fp32."""
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    rows = x.size // d if d else 0
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    _load().oracle_quantize_e4m3_rows(_ptr(x), rows, d, _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize_e4m3_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """scale[r] * E4M3(codes[r, i]) in fp64 (exact)."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    d = codes.shape[-1]
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_dequantize_e4m3_rows(_ptr(codes), _ptr(scales), codes.size // d if d else 0, d, _ptr(out))
    return out


def quantize_i8_rows(x: np.ndarray):
    """Rows x[..., d] (fp32 values; bf16 bits may be given as uint16) -> (codes
    int8 [..., d], scales float32 [...]): scale = amax / 127 and codes the
    nearest integers to x * (1 / scale), ties to even, decided in fp32."""
    if x.dtype == np.uint16:
        x = (x.astype(np.uint32) << 16).view(np.float32)
    x = np.ascontiguousarray(x, dtype=np.float32)
    d = x.shape[-1]
    rows = x.size // d if d else 0
    codes = np.empty(x.shape, dtype=np.int8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    _load().oracle_quantize_i8_rows(_ptr(x), rows, d, _ptr(codes), _ptr(scales))
    return codes, scales


def dequantize_i8_rows(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """scale[r] * codes[r, i] in fp64 (exact)."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    scales = np.ascontiguousarray(scales, dtype=np.float32)
    d = codes.shape[-1]
    out = np.empty(codes.shape, dtype=np.float64)
    _load().oracle_dequantize_i8_rows(_ptr(codes), _ptr(scales), codes.size // d if d else 0, d, _ptr(out))
    return out


_CODECS = {"fp8": (quantize_e4m3_rows, dequantize_e4m3_rows), "int8": (quantize_i8_rows, dequantize_i8_rows)}


# ---------------------------------------------------------------------------
# prefill over an FP8 cache (inference-optimisation page §11.7, a chunk of new
# tokens after a cached prefix, with §15.5.1's quantised K/V): the new rows are
# quantised into the cache exactly as the append quantises them, and every
# cached row, old or new, stands for scale * E4M3(code).  Attention is then
# the plain definition over those values.  Composed only of the functions
# above (quantiser, indexed copies, decoder, attention).
# ---------------------------------------------------------------------------

def fp8_cache_after_append(codes: np.ndarray, scales: np.ndarray, new_rows: np.ndarray, start_pos,
                           block_table=None, codec: str = "fp8"):
    """(codes, scales) of an FP8 (or, with codec="int8", INT8) cache after the
    quantising append of new_rows [B, s, K, d] (bf16 bits or fp32) at
    start_pos: codes [B,K,S,d] / [N,K,bs,d] uint8 (int8), scales [B,K,S] /
    [N,K,bs] float32."""
    qc, qs = _CODECS[codec][0](new_rows)
    codes = np.ascontiguousarray(codes).copy()
    scales = np.ascontiguousarray(scales, dtype=np.float32).copy()
    sc4, qs4 = scales[..., None], np.ascontiguousarray(qs[..., None])
    if block_table is None:
        kv_append(codes, qc, start_pos)
        kv_append(sc4, qs4, start_pos)
    else:
        kv_append_paged(codes, qc, start_pos, block_table)
        kv_append_paged(sc4, qs4, start_pos, block_table)
    return codes, sc4[..., 0]


def prefill_fp8_rows(q, k_codes, k_scales, v_codes, v_scales, start_pos, s: int, causal: bool, scale: float, rows,
                     window: int = 0, block_table=None, codec: str = "fp8") -> np.ndarray:
    """Attention rows (b, i, h) of a prefill of s new tokens over an FP8 (or
    INT8) cache that already holds them (fp8_cache_after_append): keys 0 ..
    start+s-1 of sequence b, each scale * E4M3(code) (scale * code).  q is
    [B, s, H, d] fp64."""
    kd = _CODECS[codec][1](k_codes, k_scales)
    vd = _CODECS[codec][1](v_codes, v_scales)
    start = np.asarray(start_pos, dtype=np.int32)
    kv_len = start + s
    if block_table is not None:
        S = int(kv_len.max())
        kd = gather_paged(kd, block_table, kv_len, S)
        vd = gather_paged(vd, block_table, kv_len, S)
    return attention_rows(q, kd, vd, start, kv_len, causal, scale, rows, window)
