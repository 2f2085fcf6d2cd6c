"""Several new query tokens per request (append / prefill attention) on the
GPU against the fp64 oracle: query row i of a request with n new tokens sits
at position kv_len - n + i and sees the keys up to it (the last W with a
window).  Tolerances as for decode (by KV type)."""
import dataclasses

import numpy as np
import pytest

import oracle
from kvs_testlib import compare, poison_invisible, run_library
from workloads import CONFIGS, DecodeSpec, make_inputs, small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()


def _check(inp, **kw):
    o, lse = run_library(inp, **kw)
    o_ref, lse_ref = oracle.attention_reference(inp)
    return compare(o, lse, o_ref, lse_ref, inp.spec.kv_dtype)


@pytest.mark.parametrize("chunk", [0, 16, 64])
def test_append_rows_paged_bf16(chunk):
    """1, 2, 4 and 5 new tokens with 4 query heads per KV head: 4 to 20
    columns, so one or two column groups."""
    print(f"case multi bf16 chunk={chunk}", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=4, lengths=("list", [20, 300, 1000, 2049]),
                         q_len=("list", [1, 2, 4, 5]))
    _check(make_inputs(spec, poison=True), kv_chunk=chunk)


@pytest.mark.parametrize("name", ["c5_paged_fp8_b128", "c6_paged_int4_b128"])
def test_append_rows_quantised(name):
    print(f"case multi {name}", flush=True)
    spec = small_variant(name, batch=4, lengths=("list", [3, 64, 700, 1500]), q_len=("list", [3, 0, 7, 1]))
    _check(make_inputs(spec, poison=True))


def test_whole_request_prefill_and_empty_rows():
    """A request whose every token is new (n = kv_len), one with none, one
    with a single token."""
    print("case multi prefill mix", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [37, 500, 16]), q_len=("list", [37, 0, 1]))
    _check(make_inputs(spec, poison=True), kv_chunk=16)


@pytest.mark.parametrize("window", [-1, 1, 16, 100])
def test_contiguous_prefill_mha(window):
    """Llama-shaped MHA (g = 1): 300 new rows are 300 columns per KV head,
    19 column groups; causal, with and without a window."""
    print(f"case multi prefill window={window}", flush=True)
    spec = dataclasses.replace(small_variant("c3_llama2_7b_32k", lengths=("fixed", 300), q_len=("fixed", 300)),
                               window=window)
    _check(make_inputs(spec))


def test_gemma_shaped_prefill_with_window():
    print("case multi gemma prefill", flush=True)
    spec = dataclasses.replace(small_variant("c2_gemma3_1b", lengths=("fixed", 200), q_len=("fixed", 64)),
                               window=32)
    _check(make_inputs(spec))


@pytest.mark.parametrize("g", [1, 2, 8, 16])
def test_group_sizes(g):
    print(f"case multi g={g}", flush=True)
    spec = DecodeSpec("multi", 3, 2 * g, 2, 128, 16, "bf16", "bf16", 128 ** -0.5,
                      lengths=("list", [40, 333, 900]), q_len=("list", [5, 1, 9]), seed=31 + g)
    _check(make_inputs(spec, poison=True))


def test_unified_max_with_rows():
    print("case multi unified max", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [40, 333, 900]), q_len=("list", [5, 1, 9]))
    _check(make_inputs(spec, poison=True), unified_max=200.0)


@pytest.mark.timeout(600)
def test_speculative_append_full_batch():
    """The batch-64 paged workload with 4 new tokens per request, in the
    launch configuration of a full batch; every row against the oracle."""
    print("case multi full c4 q_len 4", flush=True)
    spec = dataclasses.replace(CONFIGS["c4_paged_bf16_b64"], q_len=("fixed", 4))
    inp = make_inputs(spec)
    o, lse = run_library(inp)
    o_ref, lse_ref = oracle.attention_reference(inp)
    err, rel = compare(o, lse, o_ref, lse_ref, "bf16")
    print(f"PARITY c4 q_len 4 full: max|o-o_ref|={err:.3e} lse_rel={rel:.3e}", flush=True)


@pytest.mark.parametrize("chunk", [0, 16, 64, 1024])
def test_shared_tile_kernel_split_requests(chunk):
    """3 to 4 column groups per KV head (12 and 16 rows, 4 heads per KV
    head): the shared-tile kernel, with requests split over several chunks
    and merged, next to a one-row and an empty request."""
    print(f"case multi shared-tile chunk={chunk}", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=4, lengths=("list", [20, 300, 1000, 2049]),
                         q_len=("list", [12, 1, 16, 0]))
    _check(make_inputs(spec, poison=True), kv_chunk=chunk)


@pytest.mark.parametrize("name", ["c5_paged_fp8_b128", "c6_paged_int4_b128", "c2_gemma3_1b"])
def test_shared_tile_kernel_kv_types_and_head_dims(name):
    print(f"case multi shared-tile {name}", flush=True)
    if name == "c2_gemma3_1b":  # head_dim 256: one column group per wave
        spec = small_variant(name, lengths=("fixed", 700), q_len=("fixed", 100))
        _check(make_inputs(spec), kv_chunk=128)
    else:
        spec = small_variant(name, batch=3, lengths=("list", [40, 700, 1500]), q_len=("list", [40, 9, 33]))
        _check(make_inputs(spec, poison=True), kv_chunk=256)


def test_shared_tile_long_prefill_sampled():
    """A fresh 2048-token MHA prefill (128 column groups per head) against
    the oracle on sampled rows: the first, a middle one and the last rows
    of several 128-column workgroups."""
    print("case multi shared-tile prefill 2048", flush=True)
    spec = small_variant("c3_llama2_7b_32k", lengths=("fixed", 2048), q_len=("fixed", 2048))
    inp = make_inputs(spec)
    o, lse = run_library(inp)
    # each sampled row r sees keys 0 .. r: decode over the first r + 1 tokens
    for r in [0, 1, 15, 127, 128, 1000, 1023, 2046, 2047]:
        one = dataclasses.replace(inp, q=inp.q[r:r + 1], qo_indptr=None, kv_len=np.array([r + 1], np.int32))
        o_ref, lse_ref = oracle.decode_reference(one)
        compare(o[r:r + 1], lse[r:r + 1], o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("q_len", [("uniform", 0, 3), ("uniform", 2, 12)])
def test_rows_large_batch_device_planned(q_len):
    """300 requests: the work list comes from kv_len on the device (scan),
    with 0-3 rows (the decode kernel) or 2-12 rows per request (the
    shared-tile kernel, up to 3 groups of 16 at 4 heads per KV head)."""
    print(f"case multi large batch {q_len}", flush=True)
    spec = DecodeSpec("bigrows", 300, 8, 2, 128, 16, "bf16", "bf16", 0.1, lengths=("uniform", 12, 700),
                      q_len=q_len, seed=41)
    inp = make_inputs(spec, poison=True)
    for chunk in (0, 64):
        _check(inp, kv_chunk=chunk)


def test_rows_many_items_device_planned():
    """More than 256 splits of one request (16-token chunks of an 8192-key
    request: the device-side work list) with 40 and 3 new rows."""
    print("case multi many items", flush=True)
    spec = DecodeSpec("itemsrows", 2, 8, 2, 128, 16, "bf16", "bf16", 0.1, lengths=("list", [8192, 300]),
                      q_len=("list", [40, 3]), seed=42)
    _check(make_inputs(spec, poison=True), kv_chunk=16)


@pytest.mark.parametrize("P", [32, 64])
@pytest.mark.parametrize("rows", [[3, 1, 5], [20, 9, 33]])
def test_rows_page_sizes(P, rows):
    print(f"case multi page {P} rows {rows}", flush=True)
    spec = DecodeSpec("pagesrows", 3, 8, 2, 128, P, "bf16", "bf16", 0.1, lengths=("list", [40, 900, 2000]),
                      q_len=("list", rows), seed=P + rows[0])
    _check(make_inputs(spec, poison=True))


@pytest.mark.parametrize("kv", ["fp8", "int4"])
@pytest.mark.parametrize("W", [1, 17, 64, 300])
def test_rows_window_quantised_32x32(W, kv):
    """fp8 and INT4 with 8 heads per KV head and 20-40 rows (the 32x32
    kernel) under a sliding window."""
    print(f"case multi window {kv} {W}", flush=True)
    name = "c5_paged_fp8_b128" if kv == "fp8" else "c6_paged_int4_b128"
    spec = dataclasses.replace(small_variant(name, batch=3, lengths=("list", [40, 700, 1500]),
                                             q_len=("list", [40, 20, 33])), window=W)
    _check(make_inputs(spec, poison=True))


@pytest.mark.parametrize("Hq,Hk,kv", [(16, 8, "bf16"), (8, 2, "bf16"), (16, 8, "int4"), (8, 2, "int4")])
def test_fresh_prefill_longer_than_a_chunk(Hq, Hk, kv):
    """A fresh 1024-row prefill in 256-key chunks: the rows reach over four
    chunks, so the multi-row kernels take their XCD-balanced workgroup order
    (whole KV heads per XCD with 8 KV heads, interleaved row blocks with 2);
    both KV types run the 32x32 kernel.  Every row against the oracle."""
    print(f"case multi fresh prefill Hq={Hq} Hk={Hk} kv={kv}", flush=True)
    spec = DecodeSpec("freshpf", 2, Hq, Hk, 128, 16, kv, "bf16", 128 ** -0.5,
                      lengths=("list", [1024, 700]), q_len=("list", [1024, 700]), seed=23 + Hk)
    _check(make_inputs(spec, poison=True), kv_chunk=256)


@pytest.mark.parametrize("name,q_len,d,window", [
    ("c4_paged_bf16_b64", 1, 128, 300),     # decode kernel, one row
    ("c5_paged_fp8_b128", 1, 128, 300),
    ("c5_paged_fp8_b128", 3, 128, 200),     # 32-column kernel (two column groups), fp8
    ("c4_paged_bf16_b64", 6, 128, 200),     # 32-column kernel, bf16
    ("c4_paged_bf16_b64", 40, 128, 250),    # 32x32 kernel, bf16
    ("c5_paged_fp8_b128", 40, 128, 250),    # 32x32 kernel, fp8
    ("c4_paged_bf16_b64", 40, 64, 250),     # shared-tile kernel (head_dim 64)
    ("c4_paged_bf16_b64", 40, 256, 250),    # 32x32 kernel, head_dim 256
    ("c5_paged_fp8_b128", 40, 256, 250),    # shared-tile kernel, fp8 at head_dim 256
])
def test_keys_before_the_window_may_be_nan(name, q_len, d, window):
    """K/V codes of keys no query sees (before the first row's window) are
    NaN: every kernel must leave them out of the result (a masked weight of
    0 times a NaN value would poison the output)."""
    print(f"case multi NaN before window {name} q={q_len} d={d} W={window}", flush=True)
    spec = dataclasses.replace(small_variant(name, batch=3, lengths=("list", [700, 1500, 333]),
                                             q_len=("fixed", q_len), window=window),
                               head_dim=d, sm_scale=d ** -0.5)
    _check(poison_invisible(make_inputs(spec, poison=True)), kv_chunk=256)


@pytest.mark.parametrize("name", ["c5_paged_fp8_b128", "c6_paged_int4_b128"])
@pytest.mark.parametrize("q_len", [("list", [40, 33, 10]), ("list", [1, 1, 1])])
def test_zero_k_scale(name, q_len):
    """A request whose fp8 or INT4 K scale is 0 (an all-zero K cache
    quantised with scale 0): every visible score is 0, so its rows average V
    uniformly over their visible keys; masked keys must still get weight 0
    (-inf times a zero scale must not become NaN).  Several rows (20 column
    groups: the 32x32 kernel, whose INT4 form folds the score offset into
    the max and the exponent) and one row (the decode kernel)."""
    print(f"case multi zero K scale {name} {q_len}", flush=True)
    spec = small_variant(name, batch=3, lengths=("list", [300, 900, 64]), q_len=q_len)
    inp = make_inputs(spec, poison=True)
    k_scale = np.array(inp.k_scale, copy=True)
    k_scale[1] = 0.0
    _check(dataclasses.replace(inp, k_scale=k_scale), kv_chunk=256)


@pytest.mark.parametrize("chunk", [0, 64])
def test_fp8_head_dim_256_rows(chunk):
    """fp8 KV at head_dim 256 with several rows per request (from 3 column
    groups the shared-tile kernel, one group per wave), split and unsplit
    chunks."""
    print(f"case multi fp8 d256 chunk={chunk}", flush=True)
    spec = dataclasses.replace(small_variant("c5_paged_fp8_b128", batch=3, lengths=("list", [40, 700, 1500]),
                                             q_len=("list", [40, 9, 33])), head_dim=256, sm_scale=1 / 16)
    _check(make_inputs(spec, poison=True), kv_chunk=chunk)


def test_int4_head_dim_256_rows_from_three_groups():
    """INT4 KV at head_dim 256 with 3 to 4 column groups (6 to 8 rows of 8
    heads): the shared-tile kernel, one group per wave."""
    print("case multi int4 d256 rows", flush=True)
    spec = dataclasses.replace(small_variant("c6_paged_int4_b128", batch=3, lengths=("list", [40, 700, 1500]),
                                             q_len=("list", [6, 8, 3])), head_dim=256, sm_scale=1 / 16)
    _check(make_inputs(spec, poison=True), kv_chunk=256)


@pytest.mark.parametrize("kv", ["fp8", "bf16", "int4"])
@pytest.mark.parametrize("chunk,window,extra", [
    (0, -1, {}), (16, -1, {}), (64, 100, {}), (0, 7, {}),
    (256, -1, {"unified_max": 40.0}), (0, -1, {"logits_soft_cap": 30.0}),
])
def test_two_groups_cols32(kv, chunk, window, extra):
    """bf16, fp8 or INT4 KV, head_dim 128, 17 to 32 (query row, head) columns
    per KV head (fp8 / INT4: 3 and 4 rows of 8 heads; bf16: 5 to 8 rows of 4
    heads; and fewer): the 32-column kernel whose waves split the keys, next
    to empty and one-row requests."""
    print(f"case multi {kv} cols32 chunk={chunk} window={window} {extra}", flush=True)
    if kv in ("fp8", "int4"):
        name = "c5_paged_fp8_b128" if kv == "fp8" else "c6_paged_int4_b128"
        spec = small_variant(name, batch=5, lengths=("list", [3, 700, 2049, 40, 0]),
                             q_len=("list", [3, 4, 4, 1, 0]), window=window)
    else:
        spec = small_variant("c4_paged_bf16_b64", batch=5, lengths=("list", [5, 700, 2049, 40, 0]),
                             q_len=("list", [5, 8, 7, 1, 0]), window=window)
    if "logits_soft_cap" in extra:
        spec = dataclasses.replace(spec, soft_cap=extra["logits_soft_cap"])
        extra = {}
    _check(make_inputs(spec, poison=True), kv_chunk=chunk, **extra)


@pytest.mark.parametrize("kv", ["fp8", "bf16", "int4"])
def test_two_groups_cols32_device_planned(kv):
    """300 requests with 3 to 4 rows of 8 heads (the device-side work list)
    on the 32-column kernel."""
    print(f"case multi {kv} cols32 large batch", flush=True)
    spec = DecodeSpec("cols32rows", 300, 16, 2, 128, 16, kv, "bf16", 128 ** -0.5,
                      lengths=("uniform", 4, 600), q_len=("uniform", 3, 4), seed=77)
    _check(make_inputs(spec, poison=True))


@pytest.mark.parametrize("rows,window", [(20, -1), (32, -1), (27, 9)])
def test_two_groups_cols32_contiguous(rows, window):
    """A contiguous MHA cache (one head per KV head) with 17 to 32 new rows:
    two column groups on the 32-column kernel over [L, Hk, d] rows."""
    print(f"case multi cols32 contiguous rows={rows} window={window}", flush=True)
    spec = small_variant("c3_llama2_7b_32k", lengths=("fixed", 1500), q_len=("fixed", rows), window=window)
    _check(make_inputs(spec), kv_chunk=256)
