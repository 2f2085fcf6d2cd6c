"""The three large workloads at full size, in the launch configuration the
benchmark times (heuristic split count, matrix-core kernel), every (request,
query head) output against the fp64 oracle over the whole batch."""
import numpy as np
import pytest

import oracle
from kvs_testlib import compare, run_library, to_torch
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _full(name):
    import torch

    print(f"case {name} full size: drawing inputs", flush=True)
    inp = make_inputs(CONFIGS[name])
    t = to_torch(inp)
    o, lse = run_library(inp, tensors=t)
    del t
    torch.cuda.empty_cache()
    print(f"case {name}: oracle over all {inp.spec.batch} requests", flush=True)
    o_ref, lse_ref = oracle.decode_reference(inp)
    err, rel = compare(o, lse, o_ref, lse_ref, inp.spec.kv_dtype)
    print(f"PARITY {name} full: max|o-o_ref|={err:.3e} lse_rel={rel:.3e}", flush=True)


@pytest.mark.timeout(600)
def test_c3_full():
    _full("c3_llama2_7b_32k")


@pytest.mark.timeout(600)
def test_c4_full():
    _full("c4_paged_bf16_b64")


@pytest.mark.timeout(600)
def test_c5_full():
    _full("c5_paged_fp8_b128")


@pytest.mark.timeout(600)
def test_c6_int4_full():
    _full("c6_paged_int4_b128")
