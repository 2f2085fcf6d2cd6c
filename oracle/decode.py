"""fp64 CPU oracle of single-query decode attention over a KV cache.

TEST INFRASTRUCTURE: only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  It shares no code with the
HIP library and never calls it.

What is computed (for request b, query head h, kv head h // g):

* the visible keys J_b = { t : lo_b <= t <= L_b - 1 }, lo_b = max(0, L_b - W)
  for a window W > 0, else 0;
* scores s_t = sm_scale * <q[b, h], K[b, t, h // g]>, soft-capped to
  c * tanh(s_t / c) when a cap c > 0 is given;
* lse = m + ln sum_t exp(s_t - m), m = max_t s_t (natural log, of the scaled
  scores);
* o = sum_t exp(s_t - lse) V[b, t, h // g];
* nothing visible: o = 0, lse = -inf.

Sources (cited by page and section):

* scaled scores, softmax, then weights times V -- "Forcing Flash Attention
  onto TPU" (socker-news/Hacker News translation), section "standard causal
  attention" (here one query row and no causal mask);
* one query against a growing K/V cache -- "Beyond the Memory Wall"
  (tiptinker.com), section "2. FlashInfer";
* GQA in single decode -- the FlashInfer-from-JAX tutorial page
  (upppp.jp), section on the three kernels (single_decode);
* paged KV cache -- "Beyond the Memory Wall", FlashInfer bullet list
  (PagedAttention);
* fp8 and INT4 KV caches -- same list (compressed KV cache; the page names
  FP8/INT4 without a layout: INT4 is read here as packed two's-complement
  nibbles with a per-(request, KV head) scale, like fp8);
* sliding (local) window -- the FlashInfer-from-JAX page, Gemma 3 section
  (local vs global attention layers); "Flashlight" explainer (gist.science),
  results (sliding-window variant).
* logit soft-capping -- named, without a formula, by the FlashInfer-from-JAX
  page (Gemma 3 section: QK-norm takes the place of Gemma 2's soft-capping)
  and by the "Flashlight" explainer (results: Softcap among the score_mod
  variants).  The reading is Gemma 2's published definition, applied to the
  scaled score: s -> c * tanh(s / c), which keeps every score inside
  (-c, c) and leaves small scores almost unchanged.

Two independent forms:

* ``attend_direct`` (O1): the definition as a direct two-pass stable
  softmax (max first, then sum of exponentials);
* ``attend_chunked`` (O2): the tiled online form of the TPU page's
  "Flash Attention in JAX" section (running max, running sum and
  accumulator; rescale factor 0 when the old max is -inf, weights 0 when
  the new max is -inf, output 0 when the sum is 0), run independently on
  each KV chunk, the chunk states then merged by log-sum-exp.  The merge
  is the same rescale applied across chunks instead of consecutive tiles;
  the "Flashlight" explainer (technical summary, semantic fusion) names the
  exp(x - y) = exp(x) / exp(y) identity that makes such rescaling exact.
  The FlashDecoding++ explainer (abeam.tech), sections "problem" and
  "asynchronous softmax and unified max value", describes the per-tile
  partial softmax followed by a synchronised update with the previous max
  and sum, which is this merge.
"""
from __future__ import annotations

import math
from typing import Callable, Iterable, List, Optional, Sequence, Tuple

import numpy as np

from .codecs import decode_codes

__all__ = [
    "kv_head_of",
    "cap_scores",
    "visible_range",
    "softmax_from_scores",
    "attend_direct",
    "chunk_state",
    "merge_states",
    "attend_chunked",
    "request_kv",
    "decode_reference",
    "decode_reference_chunked",
    "decode_reference_sampled",
]


# ----------------------------------------------------------------------------
# readings of points the pages leave open
# ----------------------------------------------------------------------------

def kv_head_of(h: int, group: int) -> int:
    """GQA: consecutive query heads share one KV head (h // group)."""
    return h // group


def visible_range(kv_len: int, window: int) -> Tuple[int, int]:
    """Keys a decode query sees: [lo, kv_len).  window = -1 means all keys;
    window W > 0 means the last W keys, the newest (current) token included."""
    if window is not None and window > 0:
        return max(0, kv_len - window), kv_len
    return 0, kv_len


# ----------------------------------------------------------------------------
# O1: the definition (direct two-pass stable softmax)
# ----------------------------------------------------------------------------

def softmax_from_scores(scores: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, float]:
    """(o, lse) for one query row given its scaled scores [n] and values [n, d]."""
    scores = np.asarray(scores, dtype=np.float64)
    values = np.asarray(values, dtype=np.float64)
    if scores.shape[0] == 0:
        return np.zeros(values.shape[1], np.float64), -math.inf
    m = float(np.max(scores))
    w = np.exp(scores - m)
    total = float(np.sum(w))
    lse = m + math.log(total)
    o = (w / total) @ values
    return o, lse


def cap_scores(scores: np.ndarray, soft_cap: float) -> np.ndarray:
    """Logit soft-capping: c * tanh(s / c) for a cap c > 0; unchanged for
    c = 0 (no cap)."""
    scores = np.asarray(scores, dtype=np.float64)
    if soft_cap and soft_cap > 0:
        return soft_cap * np.tanh(scores / soft_cap)
    return scores


def attend_direct(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float,
                  soft_cap: float = 0.0) -> Tuple[np.ndarray, float]:
    """One query row q [d] against visible keys K [n, d] and values V [n, d]."""
    scores = cap_scores(sm_scale * (np.asarray(K, np.float64) @ np.asarray(q, np.float64)), soft_cap)
    return softmax_from_scores(scores, V)


# ----------------------------------------------------------------------------
# O2: tiled online softmax per chunk, chunks merged by log-sum-exp
# ----------------------------------------------------------------------------

def chunk_state(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float,
                tile: int = 16, soft_cap: float = 0.0) -> Tuple[float, float, np.ndarray]:
    """Running (max, sum, acc) after streaming K/V tiles of one chunk."""
    d = V.shape[1]
    running_max = -math.inf
    running_sum = 0.0
    acc = np.zeros(d, np.float64)
    for t0 in range(0, K.shape[0], tile):
        k_tile = np.asarray(K[t0:t0 + tile], np.float64)
        v_tile = np.asarray(V[t0:t0 + tile], np.float64)
        scores = cap_scores(sm_scale * (k_tile @ np.asarray(q, np.float64)), soft_cap)
        new_max = max(running_max, float(np.max(scores))) if scores.size else running_max
        rescale = math.exp(running_max - new_max) if math.isfinite(running_max) else 0.0
        weights = np.exp(scores - new_max) if math.isfinite(new_max) else np.zeros_like(scores)
        running_sum = rescale * running_sum + float(np.sum(weights))
        acc = rescale * acc + weights @ v_tile
        running_max = new_max
    return running_max, running_sum, acc


def merge_states(states: Iterable[Tuple[float, np.ndarray]]) -> Tuple[np.ndarray, float]:
    """Merge per-chunk (lse_c, o_c) into (o, lse).

    M = max_c lse_c; w_c = exp(lse_c - M); lse = M + ln sum_c w_c;
    o = sum_c w_c o_c / sum_c w_c.  Chunks with lse_c = -inf weigh 0; all
    -inf gives o = 0, lse = -inf.
    """
    states = list(states)
    d = states[0][1].shape[0]
    lses = np.array([s[0] for s in states], np.float64)
    if not np.any(np.isfinite(lses)):
        return np.zeros(d, np.float64), -math.inf
    M = float(np.max(lses[np.isfinite(lses)]))
    w = np.where(np.isfinite(lses), np.exp(lses - M), 0.0)
    total = float(np.sum(w))
    o = np.zeros(d, np.float64)
    for wc, (_, oc) in zip(w, states):
        if wc != 0.0:
            o = o + wc * np.asarray(oc, np.float64)
    return o / total, M + math.log(total)


def _chunk_to_lse_o(state: Tuple[float, float, np.ndarray]) -> Tuple[float, np.ndarray]:
    m, l, acc = state
    if l > 0.0:
        return m + math.log(l), acc / l
    return -math.inf, np.zeros_like(acc)


def attend_chunked(q: np.ndarray, K: np.ndarray, V: np.ndarray, sm_scale: float,
                   chunk_sizes: Sequence[int], tile: int = 16, soft_cap: float = 0.0) -> Tuple[np.ndarray, float]:
    """O2 over consecutive chunks whose sizes sum to len(K)."""
    n = K.shape[0]
    if sum(chunk_sizes) != n:
        raise ValueError("chunk sizes must cover the visible keys exactly")
    if n == 0:
        return np.zeros(V.shape[1], np.float64), -math.inf
    states = []
    t0 = 0
    for c in chunk_sizes:
        states.append(_chunk_to_lse_o(chunk_state(q, K[t0:t0 + c], V[t0:t0 + c], sm_scale, tile, soft_cap)))
        t0 += c
    return merge_states(states)


# ----------------------------------------------------------------------------
# cache layouts
# ----------------------------------------------------------------------------

def request_kv(b: int, *, k, v, kv_len, kv_dtype: str, page_size: int,
               page_indptr=None, page_indices=None, k_scale=None, v_scale=None,
               tokens: Optional[Tuple[int, int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Logical K, V of request b as float64 [n, Hk, d] for tokens [t0, t1).

    Contiguous cache: k is [L, Hk, d].  Paged cache: k is
    [num_pages, page_size, Hk, d]; logical token t of request b sits in page
    page_indices[page_indptr[b] + t // page_size], slot t % page_size.
    fp8 and int4 codes are multiplied by the per-(request, kv head) scale.
    """
    L = int(kv_len[b])
    t0, t1 = (0, L) if tokens is None else tokens
    if page_size == 0:
        kr, vr = k[t0:t1], v[t0:t1]
    else:
        t = np.arange(t0, t1)
        pages = np.asarray(page_indices)[int(page_indptr[b]) + t // page_size]
        slots = t % page_size
        kr, vr = k[pages, slots], v[pages, slots]
    K = decode_codes(kr, kv_dtype)
    V = decode_codes(vr, kv_dtype)
    if kv_dtype in ("fp8", "int4"):
        K = K * np.asarray(k_scale, np.float64)[b][None, :, None]
        V = V * np.asarray(v_scale, np.float64)[b][None, :, None]
    return K, V


def _fields(inp):
    s = inp.spec
    return dict(k=inp.k, v=inp.v, kv_len=inp.kv_len, kv_dtype=s.kv_dtype, page_size=s.page_size,
                page_indptr=inp.page_indptr, page_indices=inp.page_indices,
                k_scale=inp.k_scale, v_scale=inp.v_scale)


def decode_reference(inp, *, form: str = "direct",
                     chunker: Optional[Callable[[int], Sequence[int]]] = None,
                     requests: Optional[Sequence[int]] = None) -> Tuple[np.ndarray, np.ndarray]:
    """(o [B, Hq, d], lse [B, Hq]) in float64 for a drawn workload.

    ``inp`` carries spec (heads, dims, dtypes, sm_scale, window), q, k, v,
    kv_len, page table and scales.  ``form`` is 'direct' (O1) or 'chunked'
    (O2, with ``chunker(n_visible) -> chunk sizes``).  ``requests`` limits
    the work to some requests (the others stay NaN).
    """
    s = inp.spec
    B, Hq, Hk, d = s.batch, s.num_qo_heads, s.num_kv_heads, s.head_dim
    g = Hq // Hk
    Q = decode_codes(inp.q, s.q_dtype).reshape(B, Hq, d)
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    f = _fields(inp)
    for b in (range(B) if requests is None else requests):
        lo, hi = visible_range(int(inp.kv_len[b]), s.window)
        K, V = request_kv(b, tokens=(lo, hi), **f)
        n = hi - lo
        for h in range(Hq):
            kh = kv_head_of(h, g)
            if form == "direct":
                o[b, h], lse[b, h] = attend_direct(Q[b, h], K[:, kh], V[:, kh], s.sm_scale, s.soft_cap)
            elif form == "chunked":
                sizes = chunker(n) if chunker is not None else [n]
                o[b, h], lse[b, h] = attend_chunked(Q[b, h], K[:, kh], V[:, kh], s.sm_scale, sizes,
                                                    soft_cap=s.soft_cap)
            else:
                raise ValueError(form)
    return o, lse


def decode_reference_chunked(inp, chunker: Callable[[int], Sequence[int]]):
    return decode_reference(inp, form="chunked", chunker=chunker)


def decode_reference_sampled(inp, picks: Sequence[Tuple[int, int]]) -> List[Tuple[np.ndarray, float]]:
    """O1 for selected (request, query head) pairs only, for full-size checks."""
    s = inp.spec
    g = s.num_qo_heads // s.num_kv_heads
    Q = decode_codes(inp.q, s.q_dtype).reshape(s.batch, s.num_qo_heads, s.head_dim)
    f = _fields(inp)
    out = []
    cache = {}
    for b, h in picks:
        if b not in cache:
            lo, hi = visible_range(int(inp.kv_len[b]), s.window)
            cache = {b: request_kv(b, tokens=(lo, hi), **f)}
        K, V = cache[b]
        kh = kv_head_of(h, g)
        out.append(attend_direct(Q[b, h], K[:, kh], V[:, kh], s.sm_scale, s.soft_cap))
    return out
