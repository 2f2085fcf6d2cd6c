"""INT4 KV cache (packed two's-complement nibbles, per-(request, KV head)
scale) on the matrix-core kernel against the fp64 oracle on the GPU.

Tolerance: max |o - o_ref| <= 2e-2, the bf16 gate.  The oracle decodes the
same codes and scales, so quantisation error is not part of the comparison;
what remains is the kernel's arithmetic, which is the bf16 path's: the
operands 136 + n are exact in bf16 (integers below 256), q is bf16, the
weights are rounded to bf16 before the P.V product and everything is
accumulated in fp32; the offsets 136 * sum(q) and 136 * sum(p) are removed
in fp32 from sums of at most a few thousand terms.  |V| <= 8/7 * amax, the
range of the bf16 workloads' N(0, 1) values.  The whole batch-128 INT4
workload is compared in tests/test_gpu_fullsize.py."""
import dataclasses

import numpy as np
import pytest

import oracle
from kvs_testlib import compare, run_library
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
    o_ref, lse_ref = oracle.decode_reference(inp)
    return compare(o, lse, o_ref, lse_ref, "int4")


@pytest.mark.parametrize("chunk", [0, 16, 48, 1024])
def test_int4_paged_ragged(chunk):
    print(f"case int4 ragged chunk={chunk}", flush=True)
    spec = small_variant("c6_paged_int4_b128", batch=5, lengths=("list", [0, 1, 17, 300, 2049]))
    err, _ = _check(make_inputs(spec, poison=True), kv_chunk=chunk)
    print(f"  max err {err:.2e}")


@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("d", [128, 256])
def test_int4_groups_and_head_dims(g, d):
    print(f"case int4 g={g} d={d}", flush=True)
    spec = DecodeSpec("int4", 2, 2 * g, 2, d, 16, "int4", "bf16", d ** -0.5, lengths=("list", [77, 600]),
                      seed=21 + g + d)
    _check(make_inputs(spec, poison=True))


@pytest.mark.parametrize("window", [1, 100, 5000])
def test_int4_window(window):
    print(f"case int4 window={window}", flush=True)
    spec = small_variant("c6_paged_int4_b128", batch=3, lengths=("list", [50, 700, 3000]), window=window)
    _check(make_inputs(spec, poison=True), kv_chunk=64)


def test_int4_contiguous_long():
    print("case int4 contiguous", flush=True)
    spec = DecodeSpec("int4c", 1, 32, 32, 128, 0, "int4", "bf16", 128 ** -0.5, lengths=("fixed", 4096), seed=5)
    _check(make_inputs(spec))
    spec = DecodeSpec("int4c256", 1, 4, 1, 256, 0, "int4", "bf16", 1 / 16, lengths=("fixed", 8192), seed=6)
    _check(make_inputs(spec))


@pytest.mark.parametrize("phi", [3.0, 200.0])
def test_int4_unified_max(phi):
    print(f"case int4 unified max {phi}", flush=True)
    spec = small_variant("c6_paged_int4_b128", batch=3, lengths=("list", [5, 900, 128]))
    _check(make_inputs(spec, poison=True), unified_max=phi)
