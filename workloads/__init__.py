"""Seeded synthetic inputs for single-query decode attention.

This module only *draws* inputs: query vectors, a KV cache (contiguous
``[kv_len, num_kv_heads, head_dim]`` or paged
``[num_pages, page_size, num_kv_heads, head_dim]``), the page table and the
per-request lengths.  It holds none of the attention arithmetic; both the
fp64 oracle and the HIP path consume what it returns, so the two see the
identical bits.

Values are returned as the raw storage codes the library reads:
``float32`` arrays for fp32, ``uint16`` bit patterns for bfloat16 and
``uint8`` bit patterns for fp8 e4m3 (OCP "fn" variant).  Rounding from the
float32 draws to the stored type uses torch's round-to-nearest-even casts
(a library routine); fp8 values are clamped to +-448 first because torch's
cast does not saturate.

Recipe (one numpy ``Generator(PCG64(SeedSequence(seed)))``; child streams
spawned in the fixed order lengths, permutation, q, k, v):

* lengths: fixed, uniform integers, or a clipped rounded log-normal;
* logical K/V for every (request, token, kv head, dim) ~ N(0, 1) in float32,
  drawn in logical token order, then scattered into the page pool through
  a seeded permutation of the pool, so a different permutation reproduces
  the identical logical cache;
* optional per-head RMS normalisation of q and k (eps 1e-6, unit weight),
  standing in for the QK-norm of a Gemma-3 style model;
* fp8: per-(request, kv head) scale = amax / 448 over that request's K (and
  separately V) values, codes = e4m3(x / scale) with saturation;
* unused slots of each request's last page are poisoned with NaN codes when
  ``poison=True`` so that any read of padding shows up.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "DecodeSpec",
    "DecodeInputs",
    "make_inputs",
    "CONFIGS",
    "AppendInputs",
    "make_append_inputs",
    "config",
    "small_variant",
    "F32",
    "BF16",
    "FP8",
    "INT4",
]

F32, BF16, FP8, INT4 = "f32", "bf16", "fp8", "int4"
_STORE = {F32: np.float32, BF16: np.uint16, FP8: np.uint8, INT4: np.uint8}
# int4 has no NaN: its padding is the largest code (7, 7), which dominates
# any score it would wrongly enter
_POISON = {F32: np.float32(np.nan).view(np.uint32), BF16: 0x7FC0, FP8: 0x7F, INT4: 0x77}
FP8_MAX = 448.0
INT4_MAX = 7.0


@dataclasses.dataclass(frozen=True)
class DecodeSpec:
    """Shape and distribution of one decode workload."""

    name: str
    batch: int
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int  # 0 = contiguous cache (batch must be 1)
    kv_dtype: str
    q_dtype: str
    sm_scale: float
    window: int = -1
    # lengths: ("fixed", L) | ("uniform", lo, hi) | ("lognormal", mu, sigma, lo, hi)
    lengths: tuple = ("fixed", 512)
    qk_rmsnorm: bool = False
    seed: int = 1000
    # new query tokens per request: ("fixed", n) | ("list", [n_b...]) | ("uniform", lo, hi);
    # each is capped at the request's kv_len (its tokens are already cached)
    q_len: tuple = ("fixed", 1)
    # logit soft-cap c (scores become c * tanh(s / c)); 0 = none
    soft_cap: float = 0.0

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads


@dataclasses.dataclass
class DecodeInputs:
    spec: DecodeSpec
    q: np.ndarray  # [batch, Hq, d] raw codes
    k: np.ndarray  # contiguous [L, Hk, d] or paged [num_pages, P, Hk, d] raw codes
    v: np.ndarray
    kv_len: np.ndarray  # int32 [batch]
    page_indptr: Optional[np.ndarray]  # int32 [batch + 1] (paged only)
    page_indices: Optional[np.ndarray]  # int32 [nnz] (paged only)
    k_scale: Optional[np.ndarray]  # float32 [batch, Hk] (fp8 and int4 only)
    v_scale: Optional[np.ndarray]
    qo_indptr: Optional[np.ndarray] = None  # int32 [batch + 1]: query rows of each request (None: one each)

    @property
    def num_pages(self) -> int:
        return 0 if self.spec.page_size == 0 else int(self.k.shape[0])


def _rng(seed: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(5)]


def _draw_lengths(spec: DecodeSpec, rng) -> np.ndarray:
    kind = spec.lengths[0]
    if kind == "fixed":
        out = np.full(spec.batch, int(spec.lengths[1]), dtype=np.int64)
    elif kind == "uniform":
        lo, hi = spec.lengths[1], spec.lengths[2]
        out = rng.integers(lo, hi, size=spec.batch, endpoint=True)
    elif kind == "lognormal":
        mu, sigma, lo, hi = spec.lengths[1:5]
        out = np.clip(np.rint(np.exp(rng.normal(mu, sigma, size=spec.batch))), lo, hi)
    elif kind == "list":
        out = np.asarray(spec.lengths[1], dtype=np.int64)
        assert out.shape == (spec.batch,)
    else:
        raise ValueError(f"unknown length law {kind!r}")
    return out.astype(np.int32)


def _to_bf16_codes(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _to_fp8_codes(x: np.ndarray) -> np.ndarray:
    import torch

    t = torch.from_numpy(np.clip(np.ascontiguousarray(x, dtype=np.float32), -FP8_MAX, FP8_MAX))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _to_int4_codes(x: np.ndarray) -> np.ndarray:
    """[..., d] float32 already divided by its scale -> [..., d/2] packed
    signed nibbles (nearest even, clamped to [-8, 7]; element 2i low)."""
    q = np.clip(np.rint(x.astype(np.float64)), -8, 7).astype(np.int64) & 0xF
    return (q[..., 0::2] | (q[..., 1::2] << 4)).astype(np.uint8)


def _rms_normalize(x: np.ndarray) -> np.ndarray:
    """Per-head RMS normalisation over the last axis, eps 1e-6, unit weight."""
    ms = np.mean(np.square(x, dtype=np.float32), axis=-1, keepdims=True, dtype=np.float32)
    return (x / np.sqrt(ms + np.float32(1e-6))).astype(np.float32)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F32:
        return np.ascontiguousarray(x, dtype=np.float32)
    if dtype == BF16:
        return _to_bf16_codes(x)
    raise ValueError(dtype)


def make_inputs(spec: DecodeSpec, seed: Optional[int] = None, *, poison: bool = False,
                permute_pages: bool = True, perm_seed: Optional[int] = None,
                lengths: Optional[np.ndarray] = None, reserve_tokens: int = 0) -> DecodeInputs:
    """Draw one seeded workload.

    ``perm_seed`` (paged only) replaces the permutation stream's seed while
    keeping every value identical; ``permute_pages=False`` lays pages out in
    logical order (identity page table).  ``lengths`` overrides the length
    draw (used by edge-case tests).  ``reserve_tokens`` gives every request
    room for that many more tokens (pages, or rows of a contiguous cache),
    filled like the padding of a last page.
    """
    seed = spec.seed if seed is None else seed
    r_len, r_perm, r_q, r_k, r_v = _rng(seed)
    if perm_seed is not None:
        r_perm = np.random.Generator(np.random.PCG64(np.random.SeedSequence(perm_seed)))
    B, Hq, Hk, d, P = spec.batch, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim, spec.page_size
    if Hq % Hk:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    kv_len = _draw_lengths(spec, r_len) if lengths is None else np.asarray(lengths, np.int32)
    if P == 0 and B != 1:
        raise ValueError("a contiguous cache holds one request")

    qo_indptr = None
    if spec.q_len == ("fixed", 1):
        q = r_q.standard_normal((B, Hq, d), dtype=np.float32)
    else:
        r_ql = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x9E])))
        kind = spec.q_len[0]
        if kind == "fixed":
            ql = np.full(B, int(spec.q_len[1]), np.int64)
        elif kind == "list":
            ql = np.asarray(spec.q_len[1], np.int64)
        elif kind == "uniform":
            ql = r_ql.integers(spec.q_len[1], spec.q_len[2], size=B, endpoint=True)
        else:
            raise ValueError(f"unknown query-length law {kind!r}")
        ql = np.minimum(ql, kv_len.astype(np.int64))
        qo_indptr = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
        q = r_q.standard_normal((int(qo_indptr[-1]), Hq, d), dtype=np.float32)
    total = int(kv_len.sum())
    k_log = r_k.standard_normal((total, Hk, d), dtype=np.float32)
    v_log = r_v.standard_normal((total, Hk, d), dtype=np.float32)
    if spec.qk_rmsnorm:
        q = _rms_normalize(q)
        k_log = _rms_normalize(k_log)

    q_codes = _store(q, spec.q_dtype)
    offs = np.concatenate([[0], np.cumsum(kv_len, dtype=np.int64)])
    k_scale = v_scale = None
    if spec.kv_dtype == INT4:
        if d % 2:
            raise ValueError("int4 rows hold an even number of elements")
        k_scale = np.ones((B, Hk), np.float32)
        v_scale = np.ones((B, Hk), np.float32)
        k_codes = np.empty(k_log.shape[:-1] + (d // 2,), np.uint8)
        v_codes = np.empty(v_log.shape[:-1] + (d // 2,), np.uint8)
        for b in range(B):
            sl = slice(offs[b], offs[b + 1])
            for src, codes, scale in ((k_log, k_codes, k_scale), (v_log, v_codes, v_scale)):
                blk = src[sl]
                if blk.shape[0] == 0:
                    continue
                amax = np.max(np.abs(blk), axis=(0, 2))
                s = np.where(amax > 0, amax / np.float32(INT4_MAX), np.float32(1.0)).astype(np.float32)
                scale[b] = s
                codes[sl] = _to_int4_codes(blk / s[None, :, None])
    elif spec.kv_dtype == FP8:
        k_scale = np.ones((B, Hk), np.float32)
        v_scale = np.ones((B, Hk), np.float32)
        k_codes = np.empty(k_log.shape, np.uint8)
        v_codes = np.empty(v_log.shape, np.uint8)
        for b in range(B):
            sl = slice(offs[b], offs[b + 1])
            for src, codes, scale in ((k_log, k_codes, k_scale), (v_log, v_codes, v_scale)):
                blk = src[sl]  # [L_b, Hk, d]
                if blk.shape[0] == 0:
                    continue
                amax = np.max(np.abs(blk), axis=(0, 2))
                s = np.where(amax > 0, amax / np.float32(FP8_MAX), np.float32(1.0)).astype(np.float32)
                scale[b] = s
                codes[sl] = _to_fp8_codes(blk / s[None, :, None])
    else:
        k_codes = _store(k_log, spec.kv_dtype)
        v_codes = _store(v_log, spec.kv_dtype)
    del k_log, v_log

    if P == 0:
        if reserve_tokens:
            pad = np.zeros((reserve_tokens,) + k_codes.shape[1:], k_codes.dtype)
            if poison:
                fill = _POISON[spec.kv_dtype]
                pad = (np.full(pad.shape, np.uint32(fill), np.uint32).view(np.float32) if spec.kv_dtype == F32
                       else np.full(pad.shape, fill, pad.dtype))
            k_codes = np.concatenate([k_codes, pad])
            v_codes = np.concatenate([v_codes, pad])
        return DecodeInputs(spec, q_codes, k_codes, v_codes, kv_len, None, None, k_scale, v_scale, qo_indptr)

    n_pages = (kv_len.astype(np.int64) + reserve_tokens + P - 1) // P
    indptr = np.concatenate([[0], np.cumsum(n_pages)]).astype(np.int32)
    N = int(indptr[-1])
    perm = r_perm.permutation(N).astype(np.int32) if permute_pages else np.arange(N, dtype=np.int32)
    store = _STORE[spec.kv_dtype]
    pool_shape = (N, P, Hk, d // 2 if spec.kv_dtype == INT4 else d)
    if poison:
        fill = _POISON[spec.kv_dtype]
        if spec.kv_dtype == F32:
            k_pool = np.full(pool_shape, np.uint32(fill), np.uint32).view(np.float32)
            v_pool = k_pool.copy()
        else:
            k_pool = np.full(pool_shape, fill, store)
            v_pool = np.full(pool_shape, fill, store)
    else:
        k_pool = np.zeros(pool_shape, store)
        v_pool = np.zeros(pool_shape, store)
    # scatter logical tokens into their pages
    for b in range(B):
        L = int(kv_len[b])
        if L == 0:
            continue
        pages = perm[indptr[b]:indptr[b + 1]]
        full, rem = divmod(L, P)
        src_k = k_codes[offs[b]:offs[b + 1]]
        src_v = v_codes[offs[b]:offs[b + 1]]
        if full:
            k_pool[pages[:full]] = src_k[:full * P].reshape((full, P) + src_k.shape[1:])
            v_pool[pages[:full]] = src_v[:full * P].reshape((full, P) + src_v.shape[1:])
        if rem:
            k_pool[pages[full], :rem] = src_k[full * P:]
            v_pool[pages[full], :rem] = src_v[full * P:]
    return DecodeInputs(spec, q_codes, k_pool, v_pool, kv_len, indptr, perm, k_scale, v_scale, qo_indptr)


# The five workloads.  Sizes follow the decode shapes the pages discuss: an
# MHA fp32 toy, a Gemma-3-1B-like single decode (GQA 4, head_dim 256, QK-norm,
# local window 512), a Llama-2-7B long-context decode, and two batched paged
# GQA decodes (bf16 and fp8 e4m3 KV).
CONFIGS = {
    "c1_mha_f32": DecodeSpec("c1_mha_f32", 1, 8, 8, 64, 0, F32, F32, 1.0 / 8.0,
                             lengths=("fixed", 512), seed=1000),
    "c2_gemma3_1b": DecodeSpec("c2_gemma3_1b", 1, 4, 1, 256, 0, BF16, BF16, 1.0 / 16.0,
                               lengths=("fixed", 8192), qk_rmsnorm=True, seed=1001),
    "c2_gemma3_1b_w512": DecodeSpec("c2_gemma3_1b_w512", 1, 4, 1, 256, 0, BF16, BF16, 1.0 / 16.0,
                                    window=512, lengths=("fixed", 8192), qk_rmsnorm=True, seed=1001),
    "c3_llama2_7b_32k": DecodeSpec("c3_llama2_7b_32k", 1, 32, 32, 128, 0, BF16, BF16,
                                   1.0 / math.sqrt(128.0), lengths=("fixed", 32768), seed=1002),
    "c4_paged_bf16_b64": DecodeSpec("c4_paged_bf16_b64", 64, 32, 8, 128, 16, BF16, BF16,
                                    1.0 / math.sqrt(128.0), lengths=("uniform", 512, 16384), seed=1003),
    "c5_paged_fp8_b128": DecodeSpec("c5_paged_fp8_b128", 128, 64, 8, 128, 16, FP8, BF16,
                                    1.0 / math.sqrt(128.0),
                                    lengths=("lognormal", math.log(4096.0), 0.8, 128, 65536), seed=1004),
    # INT4 KV (two's-complement nibbles, scale amax/7): the batch-128 shape
    # of the fp8 workload with half its KV bytes
    "c6_paged_int4_b128": DecodeSpec("c6_paged_int4_b128", 128, 64, 8, 128, 16, INT4, BF16,
                                     1.0 / math.sqrt(128.0),
                                     lengths=("lognormal", math.log(4096.0), 0.8, 128, 65536), seed=1005),
}


def config(name: str) -> DecodeSpec:
    return CONFIGS[name]


def small_variant(name: str, *, batch: Optional[int] = None, lengths: Optional[tuple] = None,
                  window: Optional[int] = None, seed: Optional[int] = None,
                  q_len: Optional[tuple] = None) -> DecodeSpec:
    """Same heads, head_dim, dtypes and layout as a named workload, smaller sizes."""
    base = CONFIGS[name]
    kw = {}
    if q_len is not None:
        kw["q_len"] = q_len
    if batch is not None:
        kw["batch"] = batch
    if lengths is not None:
        kw["lengths"] = lengths
    if window is not None:
        kw["window"] = window
    if seed is not None:
        kw["seed"] = seed
    return dataclasses.replace(base, name=base.name + "_small", **kw)



# ----------------------------------------------------------------------------
# the step before attention: QK-norm, rotary embedding, KV append
# ----------------------------------------------------------------------------

@dataclasses.dataclass
class AppendInputs:
    """One step's new tokens for every request, and the cache they join.

    ``cache`` is a DecodeInputs whose requests each have room for the new
    tokens.  Without ``qo_indptr`` each request gets one new token, at
    position kv_len[b]; with it, rows qo_indptr[b] .. qo_indptr[b+1] - 1 are
    request b's, row i at position kv_len[b] + i.
    """
    cache: DecodeInputs
    q_new: np.ndarray   # [T, Hq, d] codes of q's type (T = rows; B without qo_indptr)
    k_new: np.ndarray   # [T, Hk, d] codes of q's type
    v_new: np.ndarray   # [T, Hk, d] codes of q's type
    q_norm_weight: Optional[np.ndarray]  # float32 [d] or None (no QK-norm)
    k_norm_weight: Optional[np.ndarray]
    eps: float
    theta: float        # 0: no rotary embedding
    interleave: bool
    qo_indptr: Optional[np.ndarray] = None  # int32 [B + 1]: new token rows of each request


def make_append_inputs(spec: DecodeSpec, seed: Optional[int] = None, *, norm: bool = True,
                       theta: float = 10000.0, interleave: bool = False, eps: float = 1e-6,
                       poison: bool = False, lengths: Optional[np.ndarray] = None,
                       rows: Optional[Sequence[int]] = None) -> AppendInputs:
    """Draw a cache like make_inputs and the new tokens: q, k, v ~ N(0, 1) in
    q's storage type; QK-norm weights ~ N(1, 0.25) per dimension when
    ``norm``.  ``rows`` (one count per request, >= 0) asks for that many new
    tokens per request (a packed ragged batch, qo_indptr); without it every
    request gets one.  Each request's cache has room for its new tokens (the
    most rows of any request are reserved after every cache), filled like
    padding."""
    seed = spec.seed if seed is None else seed
    B, Hq, Hk, d = spec.batch, spec.num_qo_heads, spec.num_kv_heads, spec.head_dim
    qo_indptr = None
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        if rows.shape != (B,) or np.any(rows < 0):
            raise ValueError("rows must hold one count >= 0 per request")
        qo_indptr = np.concatenate([[0], np.cumsum(rows)]).astype(np.int32)
    T = B if qo_indptr is None else int(qo_indptr[-1])
    reserve = 1 if rows is None else max(1, int(rows.max(initial=0)))
    cache = make_inputs(spec, seed, poison=poison, lengths=lengths, reserve_tokens=reserve)
    r_q, r_k, r_v, r_w = [np.random.Generator(np.random.PCG64(s))
                          for s in np.random.SeedSequence([seed, 0xA11]).spawn(4)]
    q = r_q.standard_normal((T, Hq, d), dtype=np.float32)
    k = r_k.standard_normal((T, Hk, d), dtype=np.float32)
    v = r_v.standard_normal((T, Hk, d), dtype=np.float32)
    wq = wk = None
    if norm:
        wq = (1.0 + 0.25 * r_w.standard_normal(d)).astype(np.float32)
        wk = (1.0 + 0.25 * r_w.standard_normal(d)).astype(np.float32)
    return AppendInputs(cache, _store(q, spec.q_dtype), _store(k, spec.q_dtype), _store(v, spec.q_dtype),
                        wq, wk, float(eps), float(theta), bool(interleave), qo_indptr)
