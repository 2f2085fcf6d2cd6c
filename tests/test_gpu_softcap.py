"""Logit soft-capping (scores c * tanh(s / c)) on the GPU against the fp64
oracle, on both kernels, every KV type, windows, several query rows and the
unified max; tolerances as for plain decode."""
import dataclasses

import numpy as np
import pytest

import oracle
from kvs_testlib import compare, run_library
from workloads import CONFIGS, make_inputs, small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()


def _capped(spec, cap):
    return dataclasses.replace(spec, soft_cap=cap)


def _check(inp, **kw):
    o, lse = run_library(inp, **kw)
    if inp.qo_indptr is None:
        o_ref, lse_ref = oracle.decode_reference(inp)
    else:
        o_ref, lse_ref = oracle.attention_reference(inp)
    compare(o, lse, o_ref, lse_ref, inp.spec.kv_dtype)


@pytest.mark.parametrize("cap", [0.5, 2.0, 50.0])
@pytest.mark.parametrize("name", ["c1_mha_f32", "c2_gemma3_1b", "c2_gemma3_1b_w512", "c3_llama2_7b_32k"])
def test_contiguous(name, cap):
    print(f"case softcap {name} cap={cap}", flush=True)
    spec = _capped(small_variant(name, lengths=("fixed", 1500)), cap)
    _check(make_inputs(spec))


@pytest.mark.parametrize("cap", [1.0, 30.0])
@pytest.mark.parametrize("name", ["c4_paged_bf16_b64", "c5_paged_fp8_b128", "c6_paged_int4_b128"])
@pytest.mark.parametrize("chunk", [0, 32])
def test_paged(name, cap, chunk):
    print(f"case softcap {name} cap={cap} chunk={chunk}", flush=True)
    spec = _capped(small_variant(name, batch=5, lengths=("list", [1, 17, 300, 2000, 64])), cap)
    _check(make_inputs(spec, poison=True), kv_chunk=chunk)


def test_valu_kernel_with_bf16():
    print("case softcap valu bf16", flush=True)
    spec = _capped(small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [5, 100, 777])), 3.0)
    _check(make_inputs(spec, poison=True), algo="valu")


def test_strong_scores():
    """q scaled up 8x: uncapped scores reach ~40, the cap of 10 folds them."""
    print("case softcap strong scores", flush=True)
    spec = _capped(small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [33, 500, 1200]), ), 10.0)
    spec = dataclasses.replace(spec, sm_scale=spec.sm_scale * 8)
    _check(make_inputs(spec, poison=True))


def test_rows_and_window():
    print("case softcap rows window", flush=True)
    spec = _capped(small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [40, 333, 900]),
                                 q_len=("list", [5, 1, 9])), 4.0)
    _check(make_inputs(dataclasses.replace(spec, window=64), poison=True))


@pytest.mark.parametrize("umax", [None, 4.0, -3.0])
@pytest.mark.parametrize("name", ["c4_paged_bf16_b64", "c5_paged_fp8_b128", "c6_paged_int4_b128"])
def test_rows_32x32_kernel(name, umax):
    """9-33 rows per request (5 to 17 groups of 16 columns: the 32x32
    kernel for every KV type at head_dim 128) with a cap, a window and
    256-key chunks, with and without a unified max."""
    print(f"case softcap rows 32x32 {name} umax={umax}", flush=True)
    spec = _capped(small_variant(name, batch=3, lengths=("list", [40, 700, 1500]), q_len=("list", [20, 9, 33])),
                   4.0)
    kw = {} if umax is None else {"unified_max": umax}
    _check(make_inputs(dataclasses.replace(spec, window=300), poison=True), kv_chunk=256, **kw)


@pytest.mark.parametrize("umax", [4.0, 1.0, -3.0])
def test_unified_max(umax):
    """The cap bounds every score by c, so a unified max of c never needs
    moving; other values exercise the moving reference."""
    print(f"case softcap unified max {umax}", flush=True)
    spec = _capped(small_variant("c5_paged_fp8_b128", batch=3, lengths=("list", [40, 333, 900])), 4.0)
    _check(make_inputs(spec, poison=True), unified_max=umax)


@pytest.mark.timeout(600)
def test_full_size():
    print("case softcap full c4", flush=True)
    inp = make_inputs(_capped(CONFIGS["c4_paged_bf16_b64"], 50.0))
    o, lse = run_library(inp)
    o_ref, lse_ref = oracle.decode_reference(inp)
    err, rel = compare(o, lse, o_ref, lse_ref, "bf16")
    print(f"PARITY c4 soft cap 50 full: max|o-o_ref|={err:.3e} lse_rel={rel:.3e}", flush=True)
