"""Helpers shared by the tests: move drawn inputs to the GPU, run the library,
compare with the oracle at the tolerances of each KV type."""
from __future__ import annotations

import math
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# max |o - o_ref| over all elements, by KV storage type.  INT4 takes the
# bf16 gate: the oracle decodes the same codes, and the kernel's arithmetic
# on them is the bf16 path's (exact bf16 operands 136 + n, bf16 weights,
# fp32 accumulation).
O_TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2, "int4": 2e-2}
LSE_REL = 1e-3


def ensure_built():
    """Build libkvsplit.so when it is missing (hipcc cross-compiles on any host)."""
    import decode_attention_kv_split_amd as kvs

    if not os.path.exists(kvs.library_path()):
        subprocess.run([sys.executable, "-m", "decode_attention_kv_split_amd.build"], cwd=ROOT, check=True)
    return kvs.load_library()


def gpu_available() -> bool:
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


def to_torch(inp, device="cuda"):
    """DecodeInputs -> dict of device tensors (bit-identical)."""
    import torch

    s = inp.spec

    def codes(x, dt):
        if dt == "f32":
            return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)
        if dt == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(x, np.uint8)).to(device)

    t = dict(q=codes(inp.q, s.q_dtype), k=codes(inp.k, s.kv_dtype), v=codes(inp.v, s.kv_dtype),
             kv_len=torch.from_numpy(inp.kv_len.astype(np.int32)).to(device))
    if s.page_size:
        t["page_indptr"] = torch.from_numpy(inp.page_indptr.astype(np.int32)).to(device)
        t["page_indices"] = torch.from_numpy(inp.page_indices.astype(np.int32)).to(device)
    if s.kv_dtype in ("fp8", "int4"):
        t["k_scale"] = torch.from_numpy(inp.k_scale).to(device)
        t["v_scale"] = torch.from_numpy(inp.v_scale).to(device)
    if getattr(inp, "qo_indptr", None) is not None:
        t["qo_indptr"] = torch.from_numpy(inp.qo_indptr.astype(np.int32)).to(device)
    return t


def run_library(inp, tensors=None, **kw):
    """Run kvs_decode through the binding; returns (o float64 numpy, lse numpy)."""
    import torch
    import decode_attention_kv_split_amd as kvs

    s = inp.spec
    t = tensors if tensors is not None else to_torch(inp)
    kw.setdefault("logits_soft_cap", s.soft_cap)
    o, lse = kvs.decode(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                        page_indices=t.get("page_indices"), kv_len_host=inp.kv_len,
                        k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), sm_scale=s.sm_scale,
                        window=s.window, kv_dtype="int4" if s.kv_dtype == "int4" else None,
                        qo_indptr=t.get("qo_indptr"),
                        qo_indptr_host=getattr(inp, "qo_indptr", None), **kw)
    torch.cuda.synchronize()
    return o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy()


def compare(o, lse, o_ref, lse_ref, kv_dtype, rows=None):
    """Assert o within the KV type's max-abs tolerance and lse within 1e-3
    relative (guarded by max(1, |lse|)); -inf must match -inf exactly."""
    if rows is not None:
        o, lse = o[rows], lse[rows]
    assert np.all(np.isfinite(o)), "non-finite output"
    err = float(np.max(np.abs(o - o_ref))) if o.size else 0.0
    assert err <= O_TOL[kv_dtype], f"max |o - o_ref| = {err:.3e} > {O_TOL[kv_dtype]}"
    inf_ref = np.isneginf(lse_ref)
    np.testing.assert_array_equal(np.isneginf(lse), inf_ref)
    fin = ~inf_ref
    rel = np.abs(lse[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
    rmax = float(np.max(rel)) if rel.size else 0.0
    assert rmax <= LSE_REL, f"lse relative error {rmax:.3e} > {LSE_REL}"
    return err, rmax


# ----------------------------------------------------------------------------
# the step before attention (kvs_append)
# ----------------------------------------------------------------------------

def _codes_to_torch(x, dt, device="cuda"):
    import torch

    if dt == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, np.float32)).to(device)
    if dt == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x, np.uint8)).to(device)


def _to_codes(t, dt):
    import torch

    t = t.detach().cpu()
    if dt == "f32":
        return t.numpy().astype(np.float32)
    if dt == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.view(torch.uint8).numpy()


def run_append(ai, in_place: bool = False, tensors=None):
    """Run kvs_append on an AppendInputs; returns (dict of numpy codes
    q_out / k_pool / v_pool, the device tensors of the cache)."""
    import torch
    import decode_attention_kv_split_amd as kvs

    s = ai.cache.spec
    t = tensors if tensors is not None else to_torch(ai.cache)
    q = _codes_to_torch(ai.q_new, s.q_dtype)
    k = _codes_to_torch(ai.k_new, s.q_dtype)
    v = _codes_to_torch(ai.v_new, s.q_dtype)
    wq = None if ai.q_norm_weight is None else torch.from_numpy(ai.q_norm_weight).cuda()
    wk = None if ai.k_norm_weight is None else torch.from_numpy(ai.k_norm_weight).cuda()
    rows = None
    if ai.qo_indptr is not None:
        rows = torch.from_numpy(np.asarray(ai.qo_indptr, np.int32)).cuda()
    q_out = kvs.append(q, k, v, t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                       page_indices=t.get("page_indices"), k_scale=t.get("k_scale"), v_scale=t.get("v_scale"),
                       q_norm_weight=wq, k_norm_weight=wk, norm_eps=ai.eps, rope_theta=ai.theta,
                       rope_interleave=ai.interleave, q_out=q if in_place else None, qo_indptr=rows,
                       qo_indptr_host=ai.qo_indptr, kv_dtype="int4" if s.kv_dtype == "int4" else None)
    torch.cuda.synchronize()
    got = {"q_out": _to_codes(q_out, s.q_dtype), "k_pool": _to_codes(t["k"], s.kv_dtype),
           "v_pool": _to_codes(t["v"], s.kv_dtype)}
    return got, t


# An fp32 kernel and the fp64 oracle may round a value that lies within this
# relative distance of a tie between two codes to either neighbour.
TIE_REL = 2.0 ** -16


def check_codes(got, y, dtype, what="", mag=None):
    """Stored codes against the oracle's float64 values y (same shape).

    Each code must be the nearest-even code of y, except where y lies within
    TIE_REL * max(|y|, mag) of the midpoint between that code and a
    neighbour: there both neighbours are right for an fp32 computation.
    ``mag`` bounds the size of the terms y is computed from (a rotated
    element a c - b s carries the rounding of |a| + |b|, not of |y|).
    Returns the number of elements that took the tie allowance (at most 1%)."""
    import oracle

    got = np.asarray(got)
    y = np.asarray(y, dtype=np.float64)
    packed = dtype == "int4"  # two codes per byte
    assert got.shape[:-1] + (got.shape[-1] * (2 if packed else 1),) == y.shape, (what, got.shape, y.shape)
    scale = np.abs(y) if mag is None else np.maximum(np.abs(y), np.asarray(mag, np.float64))
    if dtype == "f32":
        err = np.abs(got.astype(np.float64) - y)
        bad = err > TIE_REL * np.maximum(scale, 1.0)
        assert not np.any(bad), f"{what}: fp32 error {float(np.max(err)):.3e}"
        return 0
    if dtype == "int4":  # packed bytes: compare the unpacked integers
        gv = oracle.int4_to_f64(got)
        wv = oracle.int4_to_f64(oracle.encode_codes(y, "int4"))
        diff = gv != wv
        if not np.any(diff):
            return 0
        mid = (gv[diff] + wv[diff]) / 2
        near_tie = (np.abs(gv[diff] - wv[diff]) == 1) & \
            (np.abs(y[diff] - mid) <= TIE_REL * np.maximum(scale[diff], 1.0))
        assert np.all(near_tie), (f"{what}: {int(np.sum(~near_tie))} INT4 codes differ away from a tie; "
                                  f"first y={y[diff][~near_tie][:4]} got={gv[diff][~near_tie][:4]}")
        n = int(np.sum(diff))
        assert n <= max(1, y.size // 100), f"{what}: {n} of {y.size} codes at ties"
        return n
    want = oracle.encode_codes(y, dtype)
    diff = got != want
    if not np.any(diff):
        return 0
    gv = oracle.decode_codes(got[diff], dtype)
    wv = oracle.decode_codes(want[diff], dtype)
    yd = y[diff]
    if dtype == "fp8":
        yd = np.clip(yd, -448.0, 448.0)
    mid = (gv + wv) / 2
    near_tie = np.abs(yd - mid) <= TIE_REL * np.maximum(scale[diff], 2.0 ** -6)
    assert np.all(near_tie), (f"{what}: {int(np.sum(~near_tie))} codes differ away from a tie; "
                              f"first y={yd[~near_tie][:4]} got={gv[~near_tie][:4]} want={wv[~near_tie][:4]}")
    n = int(np.sum(diff))
    assert n <= max(1, got.size // 100), f"{what}: {n} of {got.size} codes at ties"
    return n


def _term_size(ai, x, weight, norm):
    """|a| + |b| of the rotation pair of every element of the rows x (the
    terms whose rounding an fp32 rotation carries), |x| without rotation."""
    import oracle
    from oracle import append as A

    z = np.abs(oracle.rms_norm(x, weight, ai.eps) if norm else np.asarray(x, np.float64))
    if ai.theta <= 0:
        return z
    a, b = A._pairs(z.shape[-1], ai.interleave)
    m = np.empty_like(z)
    m[..., a] = z[..., a] + z[..., b]
    m[..., b] = m[..., a]
    return m


def check_append(ai, got):
    """Every output of kvs_append against the oracle: q_out, the new K/V
    slots of every token row, and the rest of both pools unchanged bit for
    bit."""
    import oracle

    c = ai.cache
    s = c.spec
    Hq, Hk, d = s.num_qo_heads, s.num_kv_heads, s.head_dim
    ref = oracle.append_reference(ai)
    T = ref["q_out"].shape[0]
    Q = oracle.decode_codes(ai.q_new, s.q_dtype).reshape(T, Hq, d)
    K = oracle.decode_codes(ai.k_new, s.q_dtype).reshape(T, Hk, d)
    V = oracle.decode_codes(ai.v_new, s.q_dtype).reshape(T, Hk, d)
    mq = _term_size(ai, Q, ai.q_norm_weight, ai.q_norm_weight is not None)
    mk = _term_size(ai, K, ai.k_norm_weight, ai.k_norm_weight is not None)
    mv = np.abs(V)
    if s.kv_dtype in ("fp8", "int4"):
        req = ref["req"]
        mk = mk / np.asarray(c.k_scale, np.float64)[req][:, :, None]
        mv = mv / np.asarray(c.v_scale, np.float64)[req][:, :, None]
    check_codes(got["q_out"], ref["q_out"], s.q_dtype, "q_out", mag=mq)
    raw = lambda a: a.view(np.uint32) if a.dtype == np.float32 else a
    k_pool, v_pool = got["k_pool"], got["v_pool"]
    mask = np.ones(k_pool.shape[:-2], dtype=bool)  # [rows] or [pages, page_size]
    for r, b, pos in oracle.token_rows(ai):
        row, slot = oracle.cache_slot(b, pos, s.page_size, c.page_indptr, c.page_indices)
        kk = k_pool[row] if slot is None else k_pool[row, slot]
        vv = v_pool[row] if slot is None else v_pool[row, slot]
        check_codes(kk, ref["k"][r], s.kv_dtype, f"k[{r}]", mag=mk[r])
        check_codes(vv, ref["v"][r], s.kv_dtype, f"v[{r}]", mag=mv[r])
        if slot is None:
            mask[row] = False
        else:
            mask[row, slot] = False
    assert np.array_equal(raw(k_pool)[mask], raw(np.asarray(c.k))[mask]), "K pool changed outside the new slots"
    assert np.array_equal(raw(v_pool)[mask], raw(np.asarray(c.v))[mask]), "V pool changed outside the new slots"
    return ref


# NaN codes of the stored KV formats (INT4 has none)
_NAN_CODES = {"bf16": 0x7FC0, "fp8": 0x7F}


def poison_invisible(inp):
    """A copy of the workload whose K and V codes before each request's first
    visible key (the first query row's window start) are NaN: the library
    may require only the keys some query sees to be finite, so these must
    not change any result.  Needs a window; bf16 and fp8 KV."""
    import dataclasses

    s = inp.spec
    code = _NAN_CODES[s.kv_dtype]
    k, v = np.array(inp.k, copy=True), np.array(inp.v, copy=True)
    indptr = None if inp.qo_indptr is None else np.asarray(inp.qo_indptr)
    touched = 0
    for b in range(s.batch):
        L = int(inp.kv_len[b])
        n = 1 if indptr is None else int(indptr[b + 1] - indptr[b])
        if n == 0 or s.window <= 0:
            continue
        lo = max(0, L - n - s.window + 1)  # first row's window start
        for t in range(lo):
            if s.page_size == 0:
                k[t], v[t] = code, code
            else:
                page = int(inp.page_indices[inp.page_indptr[b] + t // s.page_size])
                k[page, t % s.page_size], v[page, t % s.page_size] = code, code
        touched += lo
    assert touched > 0, "no invisible keys to poison"
    return dataclasses.replace(inp, k=k, v=v)
