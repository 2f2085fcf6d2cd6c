"""Oracle of the step before decode attention: QK-norm, rotary embedding and
the append of the new token's K/V to the cache.  float64, plain loops.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline
leg of the benchmark use this package.  Nothing in the HIP library reads it.

Sources, by page and section:
  - QK-norm: the FlashInfer-from-JAX tutorial page, Gemma 3 section: an
    RMSNorm over each head's Q and K before their dot product (it replaces
    Gemma 2's logit soft-capping).  The page gives no constants; the reading
    here is y = x / sqrt(mean(x^2) + eps) * w with a per-dimension weight w.
  - rotary positional embedding: same page, the three-kernels section
    (apply_rope rotates a packed batch) and the Gemma 3 section (local
    layers use theta = 10,000, global layers theta = 1,000,000).  The page
    does not print the rotation; this is the published RoPE definition
    (Su et al., RoFormer): dimension pair j (j = 0 .. d/2 - 1) turns by the
    angle pos * theta^(-2j/d).  Pairs are (j, j + d/2) ("rotate half", the
    default reading) or (2j, 2j + 1) (interleaved).
  - appending the new token to the growing cache, paged or contiguous, and
    fp8 / INT4 KV: "Beyond the Memory Wall", section "2. FlashInfer".  The
    reading for both: the new token is quantised with the request's existing
    per-(request, KV head) scale, nearest-even with saturation (+-448 for
    fp8, [-8, 7] for INT4).
  - several new tokens per request (a packed, ragged batch of token rows,
    as the three-kernels section's apply_rope rotates a packed batch): rows
    qo_indptr[b] .. qo_indptr[b+1] - 1 belong to request b, and its row i
    takes position kv_len[b] + i (kv_len counts the tokens cached before the
    call, the one-token reading extended); each row is rotated at its own
    position and its K/V stored there.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from .codecs import decode_codes, encode_codes

__all__ = ["rms_norm", "rope", "rope_angles", "transform_head", "append_reference", "append_codes",
           "cache_slot", "apply_append", "token_rows"]


def rms_norm(x: np.ndarray, weight: Optional[np.ndarray], eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * weight over the last axis (weight None: 1)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    y = x / np.sqrt(ms + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    return y


def rope_angles(pos: float, d: int, theta: float) -> np.ndarray:
    """Angle of each of the d/2 dimension pairs at position pos:
    pos * theta^(-2j/d)."""
    j = np.arange(d // 2, dtype=np.float64)
    return float(pos) * np.power(float(theta), -2.0 * j / d)


def _pairs(d: int, interleave: bool):
    j = np.arange(d // 2)
    return (2 * j, 2 * j + 1) if interleave else (j, j + d // 2)


def rope(x: np.ndarray, pos: float, theta: float, interleave: bool = False) -> np.ndarray:
    """Rotate each dimension pair (a, b) of x [..., d] by its angle:
    (x_a, x_b) -> (x_a cos t - x_b sin t, x_a sin t + x_b cos t)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    t = rope_angles(pos, d, theta)
    a, b = _pairs(d, interleave)
    c, s = np.cos(t), np.sin(t)
    y = np.array(x, copy=True)
    y[..., a] = x[..., a] * c - x[..., b] * s
    y[..., b] = x[..., a] * s + x[..., b] * c
    return y


def transform_head(x: np.ndarray, pos: int, weight: Optional[np.ndarray], eps: float,
                   theta: float, interleave: bool, norm: bool) -> np.ndarray:
    """QK-norm (norm=True; weight None means unit weight) then the rotary
    embedding (theta > 0) of one head."""
    y = rms_norm(x, weight, eps) if norm else np.asarray(x, dtype=np.float64)
    return rope(y, pos, theta, interleave) if theta > 0 else y


def cache_slot(b: int, pos: int, page_size: int, page_indptr, page_indices):
    """Where token pos of request b is stored: (page, slot) of a paged cache,
    (row, None) of a contiguous one."""
    if page_size == 0:
        return pos, None
    return int(np.asarray(page_indices)[int(page_indptr[b]) + pos // page_size]), pos % page_size


def token_rows(ai):
    """(row, request, position) of every new token: one row per request at
    position kv_len[b] without qo_indptr; with it, row qo_indptr[b] + i of
    request b at position kv_len[b] + i."""
    c = ai.cache
    kv_len = np.asarray(c.kv_len, dtype=np.int64)
    B = c.spec.batch
    indptr = np.arange(B + 1) if getattr(ai, "qo_indptr", None) is None else np.asarray(ai.qo_indptr, np.int64)
    out = []
    for b in range(B):
        for i in range(int(indptr[b + 1] - indptr[b])):
            out.append((int(indptr[b]) + i, b, int(kv_len[b]) + i))
    return out


def append_reference(ai) -> dict:
    """float64 results of the pre-attention step for every new token row:
    q_out [T, Hq, d], k [T, Hk, d], v [T, Hk, d] before rounding to storage,
    the position each row takes and its request (T = rows; one per request
    without qo_indptr).  For an fp8 or INT4 cache, k and v are returned
    divided by their request's scales (the values whose nearest codes are
    stored)."""
    c = ai.cache
    s = c.spec
    Hq, Hk, d = s.num_qo_heads, s.num_kv_heads, s.head_dim
    rows = token_rows(ai)
    T = len(rows) if getattr(ai, "qo_indptr", None) is not None else s.batch
    Q = decode_codes(ai.q_new, s.q_dtype).reshape(T, Hq, d)
    K = decode_codes(ai.k_new, s.q_dtype).reshape(T, Hk, d)
    V = decode_codes(ai.v_new, s.q_dtype).reshape(T, Hk, d)
    q_out = np.empty((T, Hq, d))
    k_out = np.empty((T, Hk, d))
    v_out = np.array(V, copy=True)
    pos = np.empty(T, dtype=np.int64)
    req = np.empty(T, dtype=np.int64)
    for r, b, p in rows:
        pos[r], req[r] = p, b
        for h in range(Hq):
            q_out[r, h] = transform_head(Q[r, h], p, ai.q_norm_weight, ai.eps, ai.theta,
                                         ai.interleave, ai.q_norm_weight is not None)
        for h in range(Hk):
            k_out[r, h] = transform_head(K[r, h], p, ai.k_norm_weight, ai.eps, ai.theta,
                                         ai.interleave, ai.k_norm_weight is not None)
    if s.kv_dtype in ("fp8", "int4"):
        k_out = k_out / np.asarray(c.k_scale, np.float64)[req][:, :, None]
        v_out = v_out / np.asarray(c.v_scale, np.float64)[req][:, :, None]
    return {"q_out": q_out, "k": k_out, "v": v_out, "pos": pos, "req": req}


def append_codes(ref: dict, q_dtype: str, kv_dtype: str) -> dict:
    """Storage codes of the reference: q_out in q's type, k and v in the
    cache's type (nearest-even; fp8 and INT4 saturating)."""
    return {"q_out": encode_codes(ref["q_out"], q_dtype), "k": encode_codes(ref["k"], kv_dtype),
            "v": encode_codes(ref["v"], kv_dtype)}


def apply_append(ai, codes: dict):
    """Copies of the K and V pools with every new token row stored at its
    position; returns (k_pool, v_pool, kv_len + rows of each request)."""
    c = ai.cache
    s = c.spec
    k_pool, v_pool = np.array(c.k, copy=True), np.array(c.v, copy=True)
    kv_len = np.asarray(c.kv_len, np.int32).copy()
    for r, b, pos in token_rows(ai):
        row, slot = cache_slot(b, pos, s.page_size, c.page_indptr, c.page_indices)
        if slot is None:
            k_pool[row], v_pool[row] = codes["k"][r], codes["v"][r]
        else:
            k_pool[row, slot], v_pool[row, slot] = codes["k"][r], codes["v"][r]
        kv_len[b] += 1
    return k_pool, v_pool, kv_len
