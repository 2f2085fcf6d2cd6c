"""kvs_decode_noalloc (the entry point for callers that cannot allocate)
against kvs_decode with a caller workspace: the same kernels on the same
plan, so every output must match bit for bit (and both the fp64 oracle at
the KV type's tolerance), on two calls in a row, the second smaller."""
import numpy as np
import pytest

import oracle
from kvs_testlib import compare, to_torch
from workloads import DecodeSpec, make_inputs, small_variant

pytestmark = pytest.mark.gpu


def _both(inp, kv_chunk):
    import torch
    import decode_attention_kv_split_amd as kvs

    s = inp.spec
    t = to_torch(inp)
    common = dict(page_indptr=t.get("page_indptr"), page_indices=t.get("page_indices"), kv_len_host=inp.kv_len,
                  k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), sm_scale=s.sm_scale, window=s.window,
                  kv_chunk=kv_chunk, kv_dtype="int4" if s.kv_dtype == "int4" else None)
    stream = torch.cuda.current_stream().cuda_stream
    a1, keep1 = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], **common)
    plan = kvs.kvs_decode_plan(a1)
    assert plan.needs_merge and 0 < plan.workspace_bytes <= kvs.KVS_NOALLOC_SCRATCH_BYTES
    assert kvs.kvs_decode_noalloc(a1, stream) == kvs.KVS_OK
    a2, keep2 = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], **common)
    ws = torch.zeros(plan.workspace_bytes, dtype=torch.uint8, device="cuda")  # counters start at zero
    assert kvs.kvs_decode(a2, ws.data_ptr(), ws.numel(), stream) == kvs.KVS_OK
    torch.cuda.synchronize()
    (o1, l1), (o2, l2) = keep1[1:3], keep2[1:3]
    assert torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1,
                       o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2)
    assert torch.equal(l1, l2)
    o_ref, lse_ref = oracle.decode_reference(inp)
    return compare(o1.double().cpu().numpy(), l1.double().cpu().numpy(), o_ref, lse_ref, s.kv_dtype)


def test_noalloc_matches_workspace_call_twice():
    print("case noalloc: 300 requests (device-side work list), then 3 requests in 16-key chunks", flush=True)
    big = DecodeSpec("noalloc_big", 300, 16, 4, 128, 16, "bf16", "bf16", 128 ** -0.5, window=700,
                     lengths=("uniform", 0, 2000), seed=91)
    err, _ = _both(make_inputs(big, poison=True), kv_chunk=64)
    print(f"  first call max err {err:.2e}", flush=True)
    small = small_variant("c5_paged_fp8_b128", batch=3, lengths=("list", [40, 1, 900]))
    err, _ = _both(make_inputs(small, poison=True), kv_chunk=16)
    print(f"  second call max err {err:.2e}", flush=True)


def test_noalloc_rejects_a_call_larger_than_its_array():
    import decode_attention_kv_split_amd as kvs
    import torch

    # 16-key chunks of 18000 keys x 64 query heads x 256 dims of fp16 partials: about 37 MB
    spec = DecodeSpec("noalloc_big", 1, 64, 4, 256, 0, "bf16", "bf16", 0.1, lengths=("fixed", 18000), seed=3)
    inp = make_inputs(spec)
    t = to_torch(inp)
    a, keep = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], kv_len_host=inp.kv_len, kv_chunk=16)
    assert kvs.kvs_decode_plan(a).workspace_bytes > kvs.KVS_NOALLOC_SCRATCH_BYTES
    assert kvs.kvs_decode_noalloc(a, torch.cuda.current_stream().cuda_stream) == kvs.KVS_ERR_TOO_LARGE
