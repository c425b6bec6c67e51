"""Multi-token paged attention (prefill, chunked prefill, verifying several
draft tokens), plain fp64 -- TEST INFRASTRUCTURE ONLY.

The pages name the steps next to decode without a kernel for them: "vLLM 与
PagedAttention" section 六 ("关键的工程优化": a long prompt's prefill cut into
chunks and scheduled together with decode) and "指南" ("Chunked Prefill";
"Speculative Decoding": the large model checks several drafted tokens in one
pass).  The computation is ordinary causal attention over the request's
paged history, which is what this module writes out: for request s with
context_lens[s] = L tokens in its blocks (the chunk's own tokens included,
appended first) and n query rows, query row i sits at position p = L - n + i
and attends the tokens 0..p:

    out[i, h] = sum_{t <= p} softmax_t(scale * q[i, h] . K[t, g]) V[t, g],  g = h / (Hq / Hkv)

A query row with no token to attend (p < 0, only when n > L) is zero.  Rows
of request s are q[query_start[s] : query_start[s + 1]].  K/V are gathered
through the table ([VP] 二 "PagedAttention 的解法") in the pages' layout
[num_blocks, block_size, Hkv, D], decoded exactly to fp64; the scores are one
matrix product per (request, head), then a max pass, the exponentials, their
sum and one more product -- no blocking, no online rescaling.
"""
from __future__ import annotations

import numpy as np

from .oracle import decode_elements


def paged_prefill(q, k_cache, v_cache, block_tables, context_lens, query_start, scale, dtype) -> np.ndarray:
    q64 = decode_elements(q, dtype)                    # [total_q, Hq, D]
    k64 = decode_elements(k_cache, dtype)              # [NB, bs, Hkv, D]
    v64 = decode_elements(v_cache, dtype)
    total_q, Hq, D = q64.shape
    bs, Hkv = k64.shape[1], k64.shape[2]
    G = Hq // Hkv
    scale = float(np.float32(scale))
    out = np.zeros((total_q, Hq, D), dtype=np.float64)
    for s in range(len(context_lens)):
        L = int(context_lens[s])
        q0, q1 = int(query_start[s]), int(query_start[s + 1])
        n = q1 - q0
        if n == 0 or L <= 0:
            continue
        phys = np.array([block_tables[s, t // bs] for t in range(L)])
        off = np.arange(L) % bs
        K = k64[phys, off]                              # [L, Hkv, D]
        V = v64[phys, off]
        pos = L - n + np.arange(n)                      # position of each query row
        allowed = np.arange(L)[None, :] <= pos[:, None]  # [n, L]
        for h in range(Hq):
            g = h // G
            scores = scale * (q64[q0:q1, h] @ K[:, g].T)  # [n, L]
            scores = np.where(allowed, scores, -np.inf)
            m = scores.max(axis=1, keepdims=True)
            has = np.isfinite(m[:, 0])
            w = np.where(allowed, np.exp(scores - np.where(np.isfinite(m), m, 0.0)), 0.0)
            z = w.sum(axis=1, keepdims=True)
            o = (w @ V[:, g]) / np.where(z > 0, z, 1.0)
            out[q0:q1, h] = np.where(has[:, None], o, 0.0)
    return out
