"""Seeded synthetic inputs for grouped-query attention.

This module only draws inputs.  It holds none of the attention arithmetic;
the tests, the smoke check and the bench all take their inputs from here, and
the same arrays go to the GPU library and to the CPU oracle.

Recipe (fixed so that every run sees the same bits):

* ``numpy.random.Generator(PCG64(seed))`` with ``seed = 1000 + config id``;
* draw order: context lengths, then the block permutation (paged only), then
  Q, then K, then V; each of Q, K, V takes one 63-bit seed from that
  generator and is filled in 2^24-element chunks, chunk c drawn from
  ``PCG64(tensor seed).jumped(c)``;
* values are ``standard_normal(float32)`` (times 0.5 for the causal-prefill
  workload), rounded to bf16 with round-to-nearest-even for the bf16
  workloads, kept as fp32 for the fp32 workloads;
* cache slots that hold no token (positions >= ctx in a contiguous cache, the
  tail of a sequence's last 16-token block, pool blocks no sequence owns) hold
  a sentinel: a quiet NaN for parity runs, zero for timing runs.

The shapes follow the model shapes the pages discuss: Llama-2-70B
(H=64, K=8, d=128) and Llama-3-8B / Mistral-7B (H=32, K=8, d=128) from the
"Grouped-Query Attention" concept page (关键参数 #1-#2), and 16-token cache
blocks from the inference-optimisation page §5.4.1.
"""
from __future__ import annotations

import dataclasses
import math
import os
from typing import Optional

import numpy as np

BF16_QNAN = np.uint16(0x7FC0)
BLOCK_SIZE = 16


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str               # "decode" or "prefill"
    dtype: str              # "bf16" or "f32"
    B: int
    H: int
    K: int
    d: int
    seed: int
    ctx: tuple = ()         # decode: ("fixed", n) | ("uniform", lo, hi) | ("loguniform", lo, hi)
    s: int = 0              # prefill: query tokens per sequence
    value_scale: float = 1.0
    paged: bool = False
    block_size: int = BLOCK_SIZE
    window: int = 0         # > 0: sliding-window attention over the last `window` positions
    start: int = 0          # prefill: tokens already in the cache before the new ones
    description: str = ""

    @property
    def G(self) -> int:
        return self.H // self.K

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def S_max(self) -> int:
        """Cache capacity per sequence (the largest context the workload allows)."""
        if self.kind == "prefill":
            return self.start + self.s
        return int(self.ctx[-1])

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    "tiny_prefill_f32": Workload(
        "tiny_prefill_f32", "prefill", "f32", B=1, H=8, K=2, d=64, seed=1001, s=128,
        description="tiny causal prefill, fp32, B=1 H=8 K=2 d=64 s=128"),
    "tiny_decode_f32": Workload(
        "tiny_decode_f32", "decode", "f32", B=1, H=8, K=2, d=64, seed=1001, ctx=("fixed", 128),
        description="tiny decode, fp32, B=1 H=8 K=2 d=64, 128-token cache"),
    "llama3_8b_decode": Workload(
        "llama3_8b_decode", "decode", "bf16", B=32, H=32, K=8, d=128, seed=1002,
        ctx=("uniform", 1024, 4096),
        description="Llama-3-8B-shaped decode, bf16, B=32 H=32 K=8 d=128, ctx ~ U[1024,4096]"),
    "llama2_70b_decode": Workload(
        "llama2_70b_decode", "decode", "bf16", B=16, H=64, K=8, d=128, seed=1003,
        ctx=("fixed", 8192),
        description="Llama-2-70B-shaped decode, bf16, B=16 H=64 K=8 d=128, ctx = 8192"),
    "llama2_70b_decode_mha": Workload(
        "llama2_70b_decode_mha", "decode", "bf16", B=16, H=64, K=64, d=128, seed=1003,
        ctx=("fixed", 8192),
        description="MHA variant (K=H=64) of the Llama-2-70B decode shape"),
    "llama2_70b_decode_mqa": Workload(
        "llama2_70b_decode_mqa", "decode", "bf16", B=16, H=64, K=1, d=128, seed=1003,
        ctx=("fixed", 8192),
        description="MQA variant (K=1) of the Llama-2-70B decode shape"),
    "causal_prefill_4k": Workload(
        "causal_prefill_4k", "prefill", "bf16", B=4, H=32, K=8, d=128, seed=1004, s=4096,
        value_scale=0.5,
        description="causal prefill, bf16, B=4 H=32 K=8 d=128 s=4096, values x0.5"),
    "paged_long_decode": Workload(
        "paged_long_decode", "decode", "bf16", B=64, H=64, K=8, d=128, seed=1005,
        ctx=("loguniform", 512, 32768), paged=True,
        description="paged decode, bf16, B=64 H=64 K=8 d=128, ctx log-uniform in "
                    "[512,32768], 16-token blocks, shuffled block table"),
    # the two steps beside the hot path: a sliding-window decode with the
    # window the inference-optimisation page (§6.4.1) gives for Mistral 7B,
    # and a chunk of new tokens prefilled after a cached prefix into a paged
    # cache (§11.7's chunked prefill)
    "mistral_7b_window_decode": Workload(
        "mistral_7b_window_decode", "decode", "bf16", B=32, H=32, K=8, d=128, seed=1006,
        ctx=("fixed", 16384), window=4096,
        description="Mistral-7B-shaped sliding-window decode, bf16, B=32 H=32 K=8 d=128, ctx = 16384, "
                    "window 4096"),
    # the d = 64 head size (the vector-ALU decode kernel): the Llama-3-8B
    # decode's batch and head counts with half the head dimension
    "d64_decode": Workload(
        "d64_decode", "decode", "bf16", B=32, H=32, K=8, d=64, seed=1008,
        ctx=("uniform", 1024, 4096),
        description="decode at head size 64, bf16, B=32 H=32 K=8 d=64, ctx ~ U[1024,4096]"),
    "chunked_prefill_paged": Workload(
        "chunked_prefill_paged", "prefill", "bf16", B=4, H=32, K=8, d=128, seed=1007, s=512, start=3584,
        value_scale=0.5, paged=True,
        description="chunked prefill, bf16, B=4 H=32 K=8 d=128: 512 new tokens after a 3584-token cached "
                    "prefix, 16-token paged cache"),
}


# ---------------------------------------------------------------------------
# value encoding
# ---------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); returns uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    out = ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16))
    out = out.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_QNAN
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_CHUNK = 1 << 24


def _normal(rng: np.random.Generator, shape, dtype: str, scale: float) -> np.ndarray:
    """standard_normal(float32) * scale, stored as bf16 bits or fp32.

    One 63-bit seed is drawn from ``rng`` per tensor; the tensor is filled in
    2^24-element chunks, chunk c from ``PCG64(seed).jumped(c)``, so the chunks
    can be drawn in parallel and the result does not depend on the thread
    count."""
    n = int(np.prod(shape))
    seed = int(rng.integers(0, 2**63 - 1))
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(c):
        s0 = c * _CHUNK
        m = min(_CHUNK, n - s0)
        g = np.random.Generator(np.random.PCG64(seed).jumped(c))
        x = g.standard_normal(m, dtype=np.float32)
        if scale != 1.0:
            x *= np.float32(scale)
        out[s0:s0 + m] = f32_to_bf16_bits(x) if dtype == "bf16" else x

    chunks = (n + _CHUNK - 1) // _CHUNK
    if chunks <= 1:
        for c in range(chunks):
            fill(c)
    else:
        import concurrent.futures
        workers = max(1, min(16, os.cpu_count() or 1, chunks))
        with concurrent.futures.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(chunks)))
    return out.reshape(shape)


def sentinel(dtype: str, fill: str):
    if fill == "zero":
        return np.uint16(0) if dtype == "bf16" else np.float32(0.0)
    if fill == "nan":
        return BF16_QNAN if dtype == "bf16" else np.float32(np.nan)
    raise ValueError(fill)


def storage_dtype(dtype: str):
    return np.uint16 if dtype == "bf16" else np.float32


# ---------------------------------------------------------------------------
# context lengths and block tables
# ---------------------------------------------------------------------------

def draw_ctx(rng: np.random.Generator, spec: tuple, B: int) -> np.ndarray:
    kind = spec[0]
    if kind == "fixed":
        return np.full(B, int(spec[1]), dtype=np.int32)
    if kind == "uniform":
        return rng.integers(int(spec[1]), int(spec[2]), size=B, endpoint=True).astype(np.int32)
    if kind == "loguniform":
        lo, hi = int(spec[1]), int(spec[2])
        x = np.floor(np.exp(rng.uniform(math.log(lo), math.log(hi), size=B)))
        return np.clip(x, lo, hi).astype(np.int32)
    raise ValueError(spec)


def deal_blocks(rng: np.random.Generator, ctx: np.ndarray, block_size: int, slack_blocks: int = 0):
    """Shuffled physical block ids dealt to the sequences in order.

    Returns (block_table [B, max_blocks] int32 with -1 in unused entries,
    number of pool blocks)."""
    need = (ctx.astype(np.int64) + block_size - 1) // block_size
    n_pool = int(need.sum()) + int(slack_blocks)
    perm = rng.permutation(n_pool).astype(np.int32)
    max_blocks = int(need.max()) if len(need) else 0
    table = np.full((len(ctx), max(max_blocks, 1)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(need):
        table[b, :n] = perm[off:off + n]
        off += int(n)
    return table, n_pool


# ---------------------------------------------------------------------------
# workloads
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class DecodeInputs:
    wl: Workload
    ctx: np.ndarray                 # [B] int32, includes the newest token
    q: np.ndarray                   # [B,1,H,d]
    k: np.ndarray                   # contiguous [B,K,S_max,d] or pool [N,K,bs,d]
    v: np.ndarray
    block_table: Optional[np.ndarray] = None   # [B,max_blocks] int32 (paged only)
    n_blocks: int = 0

    def new_token_rows(self):
        """K/V rows of each sequence's newest token, [B,1,K,d] (what an append writes)."""
        B, K = self.wl.B, self.wl.K
        kn = np.empty((B, 1, K, self.wl.d), dtype=self.k.dtype)
        vn = np.empty_like(kn)
        for b in range(B):
            t = int(self.ctx[b]) - 1
            if self.block_table is None:
                kn[b, 0] = self.k[b, :, t]
                vn[b, 0] = self.v[b, :, t]
            else:
                blk = int(self.block_table[b, t // self.wl.block_size])
                kn[b, 0] = self.k[blk, :, t % self.wl.block_size]
                vn[b, 0] = self.v[blk, :, t % self.wl.block_size]
        return kn, vn


@dataclasses.dataclass
class PrefillInputs:
    wl: Workload
    start_pos: np.ndarray           # [B] int32
    q: np.ndarray                   # [B,s,H,d]
    k_new: np.ndarray               # [B,s,K,d]
    v_new: np.ndarray


def make_decode(wl: Workload, fill: str = "nan", ctx_override=None) -> DecodeInputs:
    if wl.kind != "decode":
        raise ValueError("not a decode workload")
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    ctx = draw_ctx(rng, wl.ctx, wl.B)
    if ctx_override is not None:
        ctx = np.asarray(ctx_override, dtype=np.int32).reshape(wl.B)
    table, n_pool = (None, 0)
    if wl.paged:
        table, n_pool = deal_blocks(rng, ctx, wl.block_size)
    q = _normal(rng, (wl.B, 1, wl.H, wl.d), wl.dtype, wl.value_scale)
    if wl.paged:
        shape = (n_pool, wl.K, wl.block_size, wl.d)
    else:
        shape = (wl.B, wl.K, max(wl.S_max, int(ctx.max())), wl.d)
    k = _normal(rng, shape, wl.dtype, wl.value_scale)
    v = _normal(rng, shape, wl.dtype, wl.value_scale)
    sent = sentinel(wl.dtype, fill)
    if wl.paged:
        used = np.zeros((n_pool, wl.block_size), dtype=bool)
        for b in range(wl.B):
            n = int(ctx[b])
            nb = (n + wl.block_size - 1) // wl.block_size
            blocks = table[b, :nb]
            used[blocks[:-1]] = True
            last = n - (nb - 1) * wl.block_size
            used[blocks[-1], :last] = True
        k.transpose(0, 2, 1, 3)[~used] = sent
        v.transpose(0, 2, 1, 3)[~used] = sent
    else:
        for b in range(wl.B):
            k[b, :, int(ctx[b]):] = sent
            v[b, :, int(ctx[b]):] = sent
    return DecodeInputs(wl, ctx, q, k, v, table, n_pool)


def make_prefill(wl: Workload) -> PrefillInputs:
    if wl.kind != "prefill":
        raise ValueError("not a prefill workload")
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    start = np.full(wl.B, wl.start, dtype=np.int32)
    q = _normal(rng, (wl.B, wl.s, wl.H, wl.d), wl.dtype, wl.value_scale)
    kn = _normal(rng, (wl.B, wl.s, wl.K, wl.d), wl.dtype, wl.value_scale)
    vn = _normal(rng, (wl.B, wl.s, wl.K, wl.d), wl.dtype, wl.value_scale)
    return PrefillInputs(wl, start, q, kn, vn)


def empty_cache(wl: Workload, fill: str = "nan", S_max: Optional[int] = None) -> np.ndarray:
    """A contiguous [B,K,S_max,d] cache holding only the sentinel."""
    S = wl.S_max if S_max is None else S_max
    return np.full((wl.B, wl.K, S, wl.d), sentinel(wl.dtype, fill), dtype=storage_dtype(wl.dtype))
