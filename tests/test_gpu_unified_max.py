"""The unified-max option (a caller-given starting reference max for every
chunk) against the fp64 oracle on the GPU: the result must not depend on
the value given, whether it bounds the scores, lies far below them (every
chunk then rescales as usual) or far above them (a still-empty chunk then
starts from its first scores)."""
import dataclasses

import pytest

import oracle
from kvs_testlib import compare, run_library
from workloads import make_inputs, small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()


@pytest.mark.parametrize("phi", [3.0, -20.0, 30.0, 200.0])
@pytest.mark.parametrize("name,lens", [
    ("c4_paged_bf16_b64", [0, 1, 17, 300, 2049]),
    ("c5_paged_fp8_b128", [5, 128, 1777]),
    ("c3_llama2_7b_32k", [1000]),
    ("c2_gemma3_1b", [3000]),
])
def test_unified_max_matches_oracle(phi, name, lens):
    print(f"case unified max {name} phi={phi}", flush=True)
    spec = small_variant(name, batch=len(lens), lengths=("list", lens))
    inp = make_inputs(spec, poison=spec.page_size > 0)
    o_ref, lse_ref = oracle.decode_reference(inp)
    for chunk in (0, 16):
        o, lse = run_library(inp, unified_max=phi, kv_chunk=chunk)
        compare(o, lse, o_ref, lse_ref, spec.kv_dtype)


@pytest.mark.parametrize("phi", [0.0, 100.0])
def test_unified_max_with_window_and_empty_chunks(phi):
    print(f"case unified max window phi={phi}", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [50, 700, 0]), window=100)
    inp = make_inputs(spec, poison=True)
    o_ref, lse_ref = oracle.decode_reference(inp)
    o, lse = run_library(inp, unified_max=phi, kv_chunk=64)
    compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("name,q_len,d", [
    ("c4_paged_bf16_b64", None, 128),   # decode kernel
    ("c5_paged_fp8_b128", None, 128),
    ("c6_paged_int4_b128", None, 128),  # two KV heads per workgroup
    ("c4_paged_bf16_b64", 6, 128),      # 32-column kernel
    ("c6_paged_int4_b128", 3, 128),
    ("c4_paged_bf16_b64", 40, 128),     # 32x32 kernel
    ("c5_paged_fp8_b128", 40, 128),
    ("c6_paged_int4_b128", 40, 128),
    ("c4_paged_bf16_b64", 40, 64),      # shared-tile kernel
    ("c5_paged_fp8_b128", 40, 256),
])
def test_reference_moves_after_a_window_start_inside_a_tile(name, q_len, d):
    """A column's keys are spread over several lanes.  A window start inside
    a tile leaves some of them with no visible key on that tile while the
    others already hold weights; a unified max of -3 under a cap of 4 then
    makes the reference move on a later tile (the one-row window start L - 301
    is key 29 of its 32-key tile, 13 of its 16-key one).  The state must count as
    non-empty in every lane of the column, or the lanes without keys so far
    would drop their share of the output (and could move their reference
    apart from the others)."""
    print(f"case unified max moving reference {name} q={q_len} d={d}", flush=True)
    kw = {} if q_len is None else {"q_len": ("fixed", q_len)}
    # only the column's last lanes see keys on the first tile; with several
    # rows the starts run through every offset
    spec = dataclasses.replace(small_variant(name, batch=3, lengths=("list", [714, 1530, 362]), window=301, **kw),
                               head_dim=d, sm_scale=d ** -0.5, soft_cap=4.0)
    inp = make_inputs(spec, poison=True)
    if inp.qo_indptr is None:
        o_ref, lse_ref = oracle.decode_reference(inp)
    else:
        o_ref, lse_ref = oracle.attention_reference(inp)
    for umax in (-3.0, 1.0):
        o, lse = run_library(inp, unified_max=umax, kv_chunk=256)
        compare(o, lse, o_ref, lse_ref, spec.kv_dtype)
