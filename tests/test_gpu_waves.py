"""Two ways for the four waves of a matrix-core decode workgroup to share its
work: one KV-head pack per wave over the whole chunk ("heads"; the four
waves read four adjacent head slices of the same token rows), or the tiles
of one pack dealt over the waves ("tiles").  Both against the fp64 oracle on
the same inputs: KV types, one or two KV heads per pack, head_dim 64 / 128 /
256, windows, soft-cap, a unified starting max, chunks from one tile per
wave to the 64-tile maximum, both merge places, a device-side work list and
empty requests."""
import dataclasses

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


def _run(inp, ws, wave_split, kv_chunk=0, merge_mode="auto", unified_max=None):
    import torch
    import decode_attention_kv_split_amd as kvs

    s = inp.spec
    t = to_torch(inp)
    a, keep = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                            page_indices=t.get("page_indices"), kv_len_host=inp.kv_len, k_scale=t.get("k_scale"),
                            v_scale=t.get("v_scale"), sm_scale=s.sm_scale, window=s.window, kv_chunk=kv_chunk,
                            kv_dtype="int4" if s.kv_dtype == "int4" else None, logits_soft_cap=s.soft_cap,
                            unified_max=unified_max, merge_mode=merge_mode, wave_split=wave_split)
    plan = kvs.kvs_decode_plan(a)
    assert plan.workspace_bytes <= ws.numel()
    assert kvs.kvs_decode(a, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream) == kvs.KVS_OK
    torch.cuda.synchronize()
    assert not np.any(ws[:kvs.KVS_WORKSPACE_COUNTER_BYTES].cpu().numpy()), "merge counters left non-zero"
    return keep[1].double().cpu().numpy(), keep[2].double().cpu().numpy(), plan


def _spec(name, **kw):
    return dataclasses.replace(small_variant(name), **kw)


# (id, spec, chunk, merge mode, unified max)
CASES = [
    ("bf16-g4", _spec("c4_paged_bf16_b64", batch=6, lengths=("list", [1, 17, 300, 1500, 4000, 0])), 0, "auto", None),
    ("bf16-g4-one-tile-per-wave", _spec("c4_paged_bf16_b64", batch=3, lengths=("list", [40, 333, 900])), 16, "kernel",
     None),
    ("bf16-g4-64-tiles", _spec("c4_paged_bf16_b64", batch=3, lengths=("list", [1024, 2049, 3000])), 1024, "in_partial",
     None),
    ("fp8-g8", _spec("c5_paged_fp8_b128", batch=5, lengths=("list", [5, 128, 700, 2600, 6000])), 0, "auto", None),
    ("fp8-g8-in-partial", _spec("c5_paged_fp8_b128", batch=4, lengths=("list", [200, 700, 1300, 2000])), 256,
     "in_partial", None),
    ("int4-pack2", _spec("c6_paged_int4_b128", batch=5, lengths=("list", [3, 130, 700, 2600, 5000])), 0, "auto", None),
    ("int4-pack2-merge-kernel", _spec("c6_paged_int4_b128", batch=3, lengths=("list", [500, 1700, 2900])), 160,
     "kernel", None),
    ("int4-d256", dataclasses.replace(_spec("c6_paged_int4_b128", batch=3, lengths=("list", [60, 900, 2100])),
                                      head_dim=256, sm_scale=1 / 16), 128, "auto", None),
    ("bf16-d256-hk4", DecodeSpec("d256hk4", 3, 16, 4, 256, 16, "bf16", "bf16", 1 / 16,
                                 lengths=("list", [33, 800, 2500]), seed=21), 0, "auto", None),
    ("bf16-d64-hk8", DecodeSpec("d64hk8", 3, 32, 8, 64, 16, "bf16", "bf16", 0.125,
                                lengths=("list", [70, 1000, 3100]), seed=22), 0, "auto", None),
    ("fp8-d64", DecodeSpec("fp8d64", 2, 64, 16, 64, 32, "fp8", "bf16", 0.125,
                                 lengths=("list", [900, 2000]), seed=23), 0, "auto", None),
    ("mha-contiguous", small_variant("c3_llama2_7b_32k", lengths=("fixed", 3000)), 0, "auto", None),
    ("window", _spec("c4_paged_bf16_b64", batch=4, lengths=("list", [50, 600, 1800, 4000]), window=333), 64,
     "auto", None),
    ("soft-cap", _spec("c5_paged_fp8_b128", batch=3, lengths=("list", [90, 1000, 2500]), soft_cap=30.0), 0, "auto",
     None),
    ("unified-max", _spec("c4_paged_bf16_b64", batch=3, lengths=("list", [90, 1000, 2500])), 0, "kernel", 4.0),
    # 300 requests: the work list is scanned on the device
    ("device-work-list", DecodeSpec("scan", 300, 32, 8, 128, 16, "bf16", "bf16", 0.1,
                                    lengths=("uniform", 0, 700), seed=24), 64, "auto", None),
]


@pytest.mark.parametrize("cid,spec,chunk,merge,umax", CASES, ids=[c[0] for c in CASES])
def test_heads_and_tiles_match_the_oracle(cid, spec, chunk, merge, umax):
    import torch

    print(f"case waves {cid} chunk={chunk} merge={merge}", flush=True)
    inp = make_inputs(spec, poison=True)
    o_ref, lse_ref = oracle.attention_reference(inp)
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    outs = {}
    for split, packs in (("heads", 4), ("tiles", 1)):
        for rep in range(2):  # twice: the merge counters must be back at zero
            o, lse, plan = _run(inp, ws, split, kv_chunk=chunk, merge_mode=merge, unified_max=umax)
            assert plan.wave_packs == packs
            err, rel = compare(o, lse, o_ref, lse_ref, spec.kv_dtype)
        outs[split] = (o, err, plan)
        print(f"  {split}: chunk {plan.kv_chunk} items {plan.items_per_kv_head} "
              f"merge_in_partial {plan.merge_in_partial} max err {err:.2e}", flush=True)
    # the automatic choice (either split, by the planner's rule)
    o, lse, plan = _run(inp, ws, "auto", kv_chunk=chunk, merge_mode=merge, unified_max=umax)
    compare(o, lse, o_ref, lse_ref, spec.kv_dtype)


def test_heads_rejected_where_it_does_not_apply():
    """One KV head (Hk / pack not a multiple of 4), several query rows per
    request, and the vector kernel: KVS_WAVES_HEADS is unsupported there;
    auto and tiles split the tiles."""
    import torch
    import decode_attention_kv_split_amd as kvs

    print("case waves rejected", flush=True)
    for spec in (small_variant("c2_gemma3_1b", lengths=("fixed", 600)),
                 small_variant("c4_paged_bf16_b64", batch=2, lengths=("list", [300, 900]), q_len=("list", [2, 3])),
                 small_variant("c1_mha_f32")):
        inp = make_inputs(spec)
        t = to_torch(inp)
        for split, want in (("heads", None), ("auto", 1), ("tiles", 1)):
            a, keep = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                                    page_indices=t.get("page_indices"), kv_len_host=inp.kv_len,
                                    sm_scale=spec.sm_scale, qo_indptr=t.get("qo_indptr"),
                                    qo_indptr_host=inp.qo_indptr, wave_split=split)
            if want is None:
                with pytest.raises(kvs.KvsError):
                    kvs.kvs_decode_plan(a)
                assert kvs.kvs_decode(a, 0, 0, torch.cuda.current_stream().cuda_stream) == kvs.KVS_ERR_UNSUPPORTED
            else:
                assert kvs.kvs_decode_plan(a).wave_packs == want
