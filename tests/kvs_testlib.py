"""Helpers shared by the tests: move drawn inputs to the GPU, run the library,
compare with the oracle at the tolerances of each KV type."""
from __future__ import annotations

import math
import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# max |o - o_ref| over all elements, by KV storage type
O_TOL = {"f32": 1e-5, "bf16": 2e-2, "fp8": 6e-2}
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
    if s.kv_dtype == "fp8":
        t["k_scale"] = torch.from_numpy(inp.k_scale).to(device)
        t["v_scale"] = torch.from_numpy(inp.v_scale).to(device)
    return t


def run_library(inp, tensors=None, **kw):
    """Run kvs_decode through the binding; returns (o float64 numpy, lse numpy)."""
    import torch
    import decode_attention_kv_split_amd as kvs

    s = inp.spec
    t = tensors if tensors is not None else to_torch(inp)
    o, lse = kvs.decode(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                        page_indices=t.get("page_indices"), kv_len_host=inp.kv_len,
                        k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), sm_scale=s.sm_scale,
                        window=s.window, **kw)
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
