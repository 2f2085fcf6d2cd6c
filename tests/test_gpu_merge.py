"""Where the splits are merged: inside the partial kernel (the workgroup that
brings a request's last split merges them all, counted with arrival
counters at the start of the workspace) or by the merge kernel.  Both
against the fp64 oracle; the counters must be zero again after every call,
so a workspace can serve calls of any shape in any order."""
import numpy as np
import pytest

import oracle
from kvs_testlib import compare, to_torch
from workloads import DecodeSpec, make_inputs, small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()


def _run(inp, ws, kv_chunk=0, merge_mode="in_partial"):
    """kvs_decode on a caller workspace, asking for the merge inside the
    partial kernel (the library falls back to the merge kernel where that
    is not possible); returns (o, lse, plan)."""
    import torch
    import decode_attention_kv_split_amd as kvs

    s = inp.spec
    t = to_torch(inp)
    a, keep = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                            page_indices=t.get("page_indices"), kv_len_host=inp.kv_len, k_scale=t.get("k_scale"),
                            v_scale=t.get("v_scale"), sm_scale=s.sm_scale, window=s.window, kv_chunk=kv_chunk,
                            kv_dtype="int4" if s.kv_dtype == "int4" else None, qo_indptr=t.get("qo_indptr"),
                            qo_indptr_host=inp.qo_indptr, merge_mode=merge_mode)
    plan = kvs.kvs_decode_plan(a)
    assert plan.workspace_bytes <= ws.numel()
    assert kvs.kvs_decode(a, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream) == kvs.KVS_OK
    torch.cuda.synchronize()
    o, lse = keep[1], keep[2]
    return o.double().cpu().numpy(), lse.double().cpu().numpy(), plan


def _counters_zero(ws):
    import decode_attention_kv_split_amd as kvs

    head = ws[:kvs.KVS_WORKSPACE_COUNTER_BYTES].cpu().numpy()
    return not np.any(head)


_REFS = {}


def _check(inp, ws, want_in_partial, kv_chunk=0):
    o, lse, plan = _run(inp, ws, kv_chunk)
    assert plan.needs_merge and plan.merge_in_partial == want_in_partial
    if id(inp) not in _REFS:
        _REFS[id(inp)] = (inp, oracle.attention_reference(inp))
    o_ref, lse_ref = _REFS[id(inp)][1]
    err, rel = compare(o, lse, o_ref, lse_ref, inp.spec.kv_dtype)
    assert _counters_zero(ws), "merge counters left non-zero"
    return err


def test_one_workspace_for_calls_of_any_shape():
    """A zeroed workspace through calls that merge in the partial kernel and
    calls that use the merge kernel (too many counters; a device-side work
    list), in alternation, some reaching counters the others do not use."""
    import torch

    print("case merge paths on one workspace", flush=True)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    fused_small = make_inputs(small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [100, 2000, 5000])),
                              poison=True)
    # 200 requests of 2 splits each x 128 KV heads: 25,600 counters, more than fit
    many_counters = make_inputs(DecodeSpec("counters", 200, 128, 128, 64, 16, "bf16", "bf16", 0.125,
                                           lengths=("uniform", 17, 32), seed=8), poison=True)
    fused_big = make_inputs(small_variant("c5_paged_fp8_b128", batch=250, lengths=("uniform", 40, 3000)),
                            poison=True)
    device_list = make_inputs(DecodeSpec("scan", 300, 8, 2, 128, 16, "bf16", "bf16", 0.1,
                                         lengths=("uniform", 20, 900), seed=9), poison=True)
    # 16-bit inline items: about 1200 items per KV head stay inline, 2000 do not
    inline_many = make_inputs(DecodeSpec("inline1200", 200, 8, 2, 128, 16, "bf16", "bf16", 0.1,
                                         lengths=("uniform", 641, 768), seed=10), poison=True)
    scan_many = make_inputs(DecodeSpec("scan2000", 250, 8, 2, 128, 16, "fp8", "bf16", 0.1,
                                       lengths=("uniform", 897, 1024), seed=11), poison=True)
    for rnd in range(2):
        _check(fused_small, ws, 1, kv_chunk=64)
        _check(many_counters, ws, 0, kv_chunk=16)
        _check(fused_big, ws, 1, kv_chunk=2048)
        _check(device_list, ws, 0, kv_chunk=64)
        _check(inline_many, ws, 1, kv_chunk=128)
        _check(scan_many, ws, 0, kv_chunk=128)
        _check(fused_small, ws, 1)


# (workload, rows per request, chunk, partial kernel): each kernel family
# merges its own splits; several rows per request put a request's columns in
# several column blocks, each with its own counter
FAMILIES = [
    ("c1_mha_f32", None, 64, "vector"),
    ("c3_llama2_7b_32k", None, 0, "decode, one request, 256 splits per head"),
    ("c4_paged_bf16_b64", None, 128, "decode"),
    ("c6_paged_int4_b128", None, 64, "decode, two INT4 heads per workgroup"),
    ("c4_paged_bf16_b64", ("list", [5, 7, 8]), 128, "32-column"),
    ("c5_paged_fp8_b128", ("list", [2, 4, 3]), 256, "32-column"),
    ("c6_paged_int4_b128", ("list", [3, 4, 2]), 64, "32-column"),
    ("c4_paged_bf16_b64", ("list", [30, 12, 0]), 128, "32x32 prefill"),
    ("c5_paged_fp8_b128", ("list", [2, 40, 0]), 256, "32x32 prefill"),
    ("c6_paged_int4_b128", ("list", [12, 6, 1]), 64, "32x32 prefill"),
    ("c2_gemma3_1b", ("fixed", 100), 128, "shared-tile (head_dim 256 bf16: 32x32 wave pairs)"),
]


@pytest.mark.parametrize("name,q_len,chunk,family", FAMILIES, ids=[f"{f[0]}-{f[3]}" for f in FAMILIES])
def test_merge_in_partial_kernel_families(name, q_len, chunk, family):
    import torch

    print(f"case merge in partial {name} {q_len} chunk={chunk} ({family})", flush=True)
    if name.startswith("c3") or name.startswith("c2"):
        spec = small_variant(name, lengths=("fixed", 8192 if name.startswith("c3") else 700), q_len=q_len)
    elif name.startswith("c1"):
        spec = small_variant(name)
    else:
        spec = small_variant(name, batch=3, lengths=("list", [700, 2500, 4000]), q_len=q_len)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    inp = make_inputs(spec, poison=True)
    for _ in range(3):  # the counters must be back at zero for the next call
        err = _check(inp, ws, 1, kv_chunk=chunk)
    print(f"  max err {err:.2e}", flush=True)


def test_int4_head_dim_256_rows_use_the_merge_kernel():
    import dataclasses
    import torch

    print("case merge kernel for INT4 d256 shared-tile", flush=True)
    spec = dataclasses.replace(small_variant("c6_paged_int4_b128", batch=3, lengths=("list", [40, 700, 1500]),
                                             q_len=("list", [6, 8, 3])), head_dim=256, sm_scale=1 / 16)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    _check(make_inputs(spec, poison=True), ws, 0, kv_chunk=256)
