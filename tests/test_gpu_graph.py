"""kvs_decode captured into a HIP graph (torch.cuda.CUDAGraph on ROCm).

A call only launches kernels: the host-planned work lists travel in the
kernel arguments and nothing is set or copied on the stream, so a captured
step must replay the eager result bit for bit (a fixed plan is
deterministic).  Each replay follows eager work on the same buffers and a
synchronisation, and every replay is checked."""
import numpy as np
import pytest

from kvs_testlib import to_torch
from workloads import make_inputs, small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()


@pytest.mark.parametrize("name,q_len", [
    ("c4_paged_bf16_b64", None),                  # decode, split requests merged
    ("c5_paged_fp8_b128", None),
    ("c4_paged_bf16_b64", ("list", [12, 40, 0])),  # several rows: the 32x32 kernel
])
def test_graph_replays_match_eager(name, q_len):
    import torch
    import decode_attention_kv_split_amd as kvs

    print(f"case graph {name} q_len={q_len}", flush=True)
    kw = dict(batch=3, lengths=("list", [40, 700, 1300]))
    if q_len is not None:
        kw["q_len"] = q_len
    spec = small_variant(name, **kw)
    inp = make_inputs(spec, poison=True)
    t = to_torch(inp)
    rows = inp.q.shape[0]
    o_dtype = torch.bfloat16 if spec.q_dtype == "bf16" else torch.float32
    dev = t["q"].device

    def call(o, lse, ws):
        kvs.decode(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                   page_indices=t.get("page_indices"), kv_len_host=inp.kv_len, k_scale=t.get("k_scale"),
                   v_scale=t.get("v_scale"), sm_scale=spec.sm_scale, window=spec.window, out=o, lse=lse,
                   workspace=ws, qo_indptr=t.get("qo_indptr"), qo_indptr_host=inp.qo_indptr)

    a, _keep = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                             page_indices=t.get("page_indices"), kv_len_host=inp.kv_len,
                             k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), sm_scale=spec.sm_scale,
                             window=spec.window, qo_indptr=t.get("qo_indptr"), qo_indptr_host=inp.qo_indptr)
    ws = torch.zeros(max(1, kvs.kvs_decode_workspace_bytes(a)), dtype=torch.uint8, device=dev)  # counters start at zero
    shape_o = (rows, spec.num_qo_heads, spec.head_dim)
    o_e = torch.empty(shape_o, dtype=o_dtype, device=dev)
    lse_e = torch.empty((rows, spec.num_qo_heads), dtype=torch.float32, device=dev)
    call(o_e, lse_e, ws)
    torch.cuda.synchronize()

    o_g, lse_g = torch.empty_like(o_e), torch.empty_like(lse_e)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up on a side stream before capture
        call(o_g, lse_g, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call(o_g, lse_g, ws)
    torch.cuda.synchronize()

    for rep in range(3):
        o_g.fill_(float("nan"))  # eager work on the same buffers between replays
        lse_g.fill_(0.0)
        ws.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        same_o = torch.equal(o_g.view(torch.int16) if o_dtype == torch.bfloat16 else o_g.view(torch.int32),
                             o_e.view(torch.int16) if o_dtype == torch.bfloat16 else o_e.view(torch.int32))
        same_lse = torch.equal(lse_g.view(torch.int32), lse_e.view(torch.int32))
        assert same_o and same_lse, f"replay {rep} differs from the eager call"
    assert np.isfinite(o_e.float().cpu().numpy()).all()
