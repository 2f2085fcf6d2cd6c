"""Oracle of attention for several new query tokens per request (append /
prefill attention over the cache), float64.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use this module.  Nothing in the HIP library reads it.

Request b has n_b new query rows, whose keys and values are already the
last n_b tokens of its cache (kv_len L_b).  Query row i sits at position
p = L_b - n_b + i and, as in the causal attention of "Forcing Flash
Attention onto TPU" (section "standard causal attention": a query attends
to keys at or before its own position), sees the keys t <= p; with a window
W > 0 only the last W of them, t >= p - W + 1 (the local layers of the
FlashInfer-from-JAX page's Gemma 3 section).  n_b = 1 is decode attention.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np

from .codecs import decode_codes
from .decode import _fields, attend_direct, kv_head_of, request_kv

__all__ = ["query_position", "query_range", "attention_reference"]


def query_position(kv_len: int, n_q: int, i: int) -> int:
    """Position of query row i of a request with n_q new tokens."""
    return kv_len - n_q + i


def query_range(kv_len: int, n_q: int, i: int, window: int) -> Tuple[int, int]:
    """Keys [lo, hi) that query row i sees."""
    p = query_position(kv_len, n_q, i)
    lo = max(0, p - window + 1) if window > 0 else 0
    return lo, p + 1


def attention_reference(inp, requests: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(o [total_q, Hq, d], lse [total_q, Hq]) for a workload with query
    rows per request given by inp.qo_indptr (None: one row per request)."""
    s = inp.spec
    B, Hq, Hk, d = s.batch, s.num_qo_heads, s.num_kv_heads, s.head_dim
    g = Hq // Hk
    indptr = np.arange(B + 1) if inp.qo_indptr is None else np.asarray(inp.qo_indptr, np.int64)
    total = int(indptr[-1])
    Q = decode_codes(inp.q, s.q_dtype).reshape(total, Hq, d)
    o = np.full((total, Hq, d), np.nan)
    lse = np.full((total, Hq), np.nan)
    f = _fields(inp)
    for b in (range(B) if requests is None else requests):
        L = int(inp.kv_len[b])
        n = int(indptr[b + 1] - indptr[b])
        if n == 0:
            continue
        K, V = request_kv(b, **f)  # all L tokens
        for i in range(n):
            lo, hi = query_range(L, n, i, s.window)
            r = int(indptr[b]) + i
            for h in range(Hq):
                kh = kv_head_of(h, g)
                o[r, h], lse[r, h] = attend_direct(Q[r, h], K[lo:hi, kh], V[lo:hi, kh], s.sm_scale, s.soft_cap)
    return o, lse
