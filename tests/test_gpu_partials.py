"""Row-scaled fp16 split partials of bf16 caches (the decode kernel stores
each split's partial row in fp16 times a power of two, and the merge
multiplies it back).  V is bf16 N(0, 1) scaled by exact powers of two, far
above fp16's largest value (2^18) and far below its smallest normal (2^-20),
and in a mix whose splits differ by 2^32 in scale; the output scales by the
same power of two, so o / 2^k must match the oracle's o / 2^k to the bf16
gate.  Forced short chunks make every request split and the launch larger
than one workgroup per CU (smaller launches keep fp32 partials); both wave
splits and both merge places."""
import dataclasses

import numpy as np
import pytest

import oracle
from kvs_testlib import O_TOL, LSE_REL, run_library
from workloads import make_inputs, small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()


def _scaled_v(inp, exps):
    """bf16 V codes times 2^exps[token] (exact: the exponent moves, the
    mantissa stays).  Paged pools: exps is indexed by the pool's token slot."""
    v = inp.v.astype(np.uint32) << 16
    f = v.view(np.float32).astype(np.float64)
    if inp.spec.page_size:
        e = np.asarray(exps, np.float64).reshape(f.shape[0], f.shape[1], 1, 1)
    else:
        e = np.asarray(exps, np.float64).reshape(f.shape[0], 1, 1)
    g = (f * np.exp2(e)).astype(np.float32)
    assert np.array_equal(g.astype(np.float64) / np.exp2(e), f), "scaling must be exact"
    return (g.view(np.uint32) >> 16).astype(np.uint16)


def _plan_format(inp, **kw):
    import decode_attention_kv_split_amd as kvs
    from kvs_testlib import to_torch

    s = inp.spec
    t = to_torch(inp)
    a, keep = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                            page_indices=t.get("page_indices"), kv_len_host=inp.kv_len, sm_scale=s.sm_scale,
                            window=s.window, qo_indptr=t.get("qo_indptr"),
                            qo_indptr_host=getattr(inp, "qo_indptr", None), **kw)
    return kvs.kvs_decode_plan(a).part_format


def _check(inp, k_out, **kw):
    import decode_attention_kv_split_amd as kvs

    assert _plan_format(inp, **kw) == kvs.KVS_PART_F16_ROWS, "the case must run the row-scaled format"
    o, lse = run_library(inp, **kw)
    o_ref, lse_ref = oracle.attention_reference(inp)
    assert np.all(np.isfinite(o)), "non-finite output"
    err = float(np.max(np.abs((o - o_ref) * 2.0 ** -k_out)))
    print(f"  max |o - o_ref| / 2^{k_out} = {err:.3e}", flush=True)
    assert err <= O_TOL["bf16"], f"max |o - o_ref| / 2^{k_out} = {err:.3e}"
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_ref))
    rel = np.abs(lse[fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
    assert float(rel.max()) <= LSE_REL


def _paged(d=128, Hq=32, Hk=8):
    spec = small_variant("c4_paged_bf16_b64", batch=5, lengths=("list", [700, 1500, 64, 3000, 17]))
    return dataclasses.replace(spec, num_qo_heads=Hq, num_kv_heads=Hk, head_dim=d)


@pytest.mark.parametrize("scale", ["big", "tiny", "mixed"])
@pytest.mark.parametrize("waves", ["tiles", "heads"])
@pytest.mark.parametrize("merge", ["kernel", "in_partial"])
def test_row_scaled_partials_paged(scale, waves, merge):
    print(f"case partials {scale} {waves} {merge}", flush=True)
    inp = make_inputs(_paged(), seed=77)
    n_pages, P = inp.v.shape[0], inp.v.shape[1]
    if scale == "big":
        exps, k_out = np.full((n_pages, P), 18.0), 18
    elif scale == "tiny":
        exps, k_out = np.full((n_pages, P), -20.0), -20
    else:  # pages alternate between 2^16 and 2^-16; one page per split, so splits differ by 2^32
        exps, k_out = np.where(np.arange(n_pages)[:, None] % 2 == 0, 16.0, -16.0) * np.ones((1, P)), 16
    inp = dataclasses.replace(inp, v=_scaled_v(inp, exps))
    # short enough for more workgroups than CUs (the launches that store row-scaled partials)
    chunk = 16 if scale == "mixed" else 32
    _check(inp, k_out, kv_chunk=chunk, wave_split=waves, merge_mode=merge)


@pytest.mark.parametrize("d,Hq,Hk", [(64, 16, 4), (256, 8, 2)])
@pytest.mark.parametrize("scale", ["big", "tiny"])
def test_row_scaled_partials_head_dims(d, Hq, Hk, scale):
    print(f"case partials d={d} {scale}", flush=True)
    inp = make_inputs(_paged(d, Hq, Hk), seed=78)
    k_out = 18 if scale == "big" else -20
    inp = dataclasses.replace(inp, v=_scaled_v(inp, np.full(inp.v.shape[:2], float(k_out))))
    _check(inp, k_out, kv_chunk=32)


def test_row_scaled_partials_contiguous_mha():
    """The 32k-token MHA decode's shape (contiguous cache, one head per KV
    head), shortened; V at 2^18."""
    print("case partials contiguous MHA", flush=True)
    spec = small_variant("c3_llama2_7b_32k", lengths=("fixed", 5000))
    inp = make_inputs(spec, seed=79)
    inp = dataclasses.replace(inp, v=_scaled_v(inp, np.full(inp.v.shape[0], 18.0)))
    _check(inp, 18, kv_chunk=64)


@pytest.mark.parametrize("d,Hq,Hk", [(128, 32, 8), (64, 16, 4)])
@pytest.mark.parametrize("scale", ["big", "tiny", "mixed"])
def test_row_scaled_partials_two_column_groups(d, Hq, Hk, scale):
    """5 to 8 query rows per request with 4 query heads per KV head: two
    groups of 16 (query row, head) columns, on the 32-column kernel (head_dim
    128) or the decode kernel's two-group form (64)."""
    print(f"case partials two groups d={d} {scale}", flush=True)
    spec = dataclasses.replace(_paged(d, Hq, Hk), q_len=("list", [8, 5, 6, 8, 1]))
    inp = make_inputs(spec, seed=80)
    n_pages, P = inp.v.shape[0], inp.v.shape[1]
    if scale == "mixed":
        exps, k_out, chunk = np.where(np.arange(n_pages)[:, None] % 2 == 0, 16.0, -16.0) * np.ones((1, P)), 16, 16
    else:
        k_out = 18 if scale == "big" else -20
        exps, chunk = np.full((n_pages, P), float(k_out)), 32
    inp = dataclasses.replace(inp, v=_scaled_v(inp, exps))
    _check(inp, k_out, kv_chunk=chunk)


@pytest.mark.parametrize("d", [128, 256])
@pytest.mark.parametrize("scale", ["big", "tiny", "mixed"])
def test_row_scaled_partials_prefill_kernel(d, scale):
    """40 query rows per request at 4 query heads per KV head (ten groups of
    16 columns): the 32x32 prefill kernel (head_dim 256: a row over a wave
    pair), planned for 16 CUs so that the launch stores row-scaled partials."""
    print(f"case partials prefill d={d} {scale}", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=5, lengths=("list", [300, 700, 64, 1200, 40]))
    spec = dataclasses.replace(spec, num_qo_heads=16 if d == 128 else 8, num_kv_heads=4 if d == 128 else 2,
                               head_dim=d, sm_scale=d ** -0.5, q_len=("list", [40, 40, 40, 40, 40]))
    inp = make_inputs(spec, seed=81)
    n_pages, P = inp.v.shape[0], inp.v.shape[1]
    if scale == "mixed":
        exps, k_out = np.where(np.arange(n_pages)[:, None] % 2 == 0, 16.0, -16.0) * np.ones((1, P)), 16
    else:
        k_out = 18 if scale == "big" else -20
        exps = np.full((n_pages, P), float(k_out))
    inp = dataclasses.replace(inp, v=_scaled_v(inp, exps))
    _check(inp, k_out, kv_chunk=64, num_cus=16)
