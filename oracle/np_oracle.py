"""Second, independent fp64 oracle in NumPy (test infrastructure only).

It restates the same definition as gqa_oracle.c without sharing any code with
it, so that the two can be checked against each other:

* ``gqa_reference``: the "Grouped-Query Attention" concept page, section
  技术原理 steps 2-4 -- reshape Q [B,s,H,d] to [B,s,K,H/K,d], attend each group
  to its own K/V head with softmax(Q_group K_g^T / sqrt(d_k)) V_g, reshape back.
  The softmax is the standard three-pass one (inference-optimisation page §9.1).

* ``online_softmax_attention``: the streaming form of the same row, written
  from the inference-optimisation page §9.2.1 (state (m, l, o); each new score
  x updates m' = max(m, x), l' = l e^(m-m') + e^(x-m'),
  o' = o e^(m-m') + v e^(x-m'); the result is o / l at the end).

* ``split_merge_attention``: the Flash-Decoding form (same page §10.2): the
  keys are cut into segments, each segment yields its own (m, l, o) and the
  segments are merged with the global max and sum.

The last two exist only to pin, in fp64, that the rewrites the GPU path uses
give the same answer as the plain definition.
"""
from __future__ import annotations

import math

import numpy as np


def visible_count(qpos: int, kv_len: int, causal: bool) -> int:
    """Keys 0..n-1 are visible; causal rows see keys j <= qpos (page §5.1)."""
    n = kv_len
    if causal:
        n = min(n, qpos + 1)
    return max(n, 0)


def gqa_reference(q, k, v, q_start, kv_len, causal: bool, scale: float, window: int = 0) -> np.ndarray:
    """q [B,Sq,H,d], k/v [B,K,Sk,d] fp64 -> out [B,Sq,H,d] fp64.
    window > 0: a row at position qpos sees keys from qpos + 1 - window on
    (sliding window, inference-optimisation page §6.4.1)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, d = q.shape
    K = k.shape[1]
    if H % K:
        raise ValueError("H must be a multiple of K")
    G = H // K
    # step 2: [B, Sq, H, d] -> [B, Sq, K, G, d]; group g holds heads g*G .. g*G+G-1
    qg = q.reshape(B, Sq, K, G, d)
    out = np.full((B, Sq, K, G, d), np.nan)
    for b in range(B):
        for i in range(Sq):
            qpos = int(q_start[b]) + i
            n = visible_count(qpos, min(int(kv_len[b]), k.shape[2]), causal)
            lo = min(max(qpos + 1 - window, 0), n) if window > 0 else 0
            if n - lo <= 0:
                continue
            for g in range(K):
                # step 3: scores of the G heads of group g against K_g
                s = scale * (qg[b, i, g] @ k[b, g, lo:n].T)       # [G, n - lo]
                m = s.max(axis=1, keepdims=True)                  # pass 1
                p = np.exp(s - m)                                 # pass 2
                out[b, i, g] = (p @ v[b, g, lo:n]) / p.sum(axis=1, keepdims=True)  # pass 3
    # step 4: back to [B, Sq, H, d]
    return out.reshape(B, Sq, H, d)


def online_softmax_row(q_row, k_rows, v_rows, scale: float):
    """One row by the streaming recurrence; returns (o / l, m, l)."""
    m = -math.inf
    l = 0.0
    o = np.zeros(v_rows.shape[1], dtype=np.float64)
    for j in range(k_rows.shape[0]):
        x = scale * float(np.dot(q_row, k_rows[j]))
        m_new = max(m, x)
        alpha = math.exp(m - m_new) if m != -math.inf else 0.0
        e = math.exp(x - m_new)
        l = l * alpha + e
        o = o * alpha + e * v_rows[j]
        m = m_new
    return o / l, m, l


def online_softmax_attention(q, k, v, q_start, kv_len, causal: bool, scale: float) -> np.ndarray:
    """Every row of gqa_reference, evaluated with the streaming recurrence."""
    q = np.asarray(q, dtype=np.float64)
    B, Sq, H, d = q.shape
    K = k.shape[1]
    G = H // K
    out = np.full(q.shape, np.nan)
    for b in range(B):
        for i in range(Sq):
            n = visible_count(int(q_start[b]) + i, min(int(kv_len[b]), k.shape[2]), causal)
            if n == 0:
                continue
            for h in range(H):
                g = h // G
                out[b, i, h], _, _ = online_softmax_row(q[b, i, h], k[b, g, :n], v[b, g, :n], scale)
    return out


def segment_partial(q_row, k_rows, v_rows, scale: float):
    """(m, l, o) of one segment: local max, local sum of exp, unnormalised V sum."""
    s = scale * (k_rows @ q_row)
    m = float(s.max())
    p = np.exp(s - m)
    return m, float(p.sum()), p @ v_rows


def merge_partials(parts):
    """Merge segment partials with the global max and sum (page §10.2)."""
    M = max(m for m, _, _ in parts)
    L = sum(l * math.exp(m - M) for m, l, _ in parts)
    O = sum(o * math.exp(m - M) for m, _, o in parts)
    return O / L


def split_merge_attention(q, k, v, kv_len, scale: float, segment: int) -> np.ndarray:
    """Decode rows (Sq == 1, attend to keys [0, kv_len)) by split-and-merge."""
    q = np.asarray(q, dtype=np.float64)
    B, Sq, H, d = q.shape
    if Sq != 1:
        raise ValueError("split_merge_attention is for one query row per sequence")
    K = k.shape[1]
    G = H // K
    out = np.full(q.shape, np.nan)
    for b in range(B):
        n = int(kv_len[b])
        for h in range(H):
            g = h // G
            parts = [segment_partial(q[b, 0, h], k[b, g, s0:min(n, s0 + segment)],
                                     v[b, g, s0:min(n, s0 + segment)], scale)
                     for s0 in range(0, n, segment)]
            out[b, 0, h] = merge_partials(parts)
    return out
