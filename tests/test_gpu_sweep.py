"""Randomized parity sweep: 150 seeded configurations drawn over KV type x
head_dim x group x KV heads x page size (or a contiguous cache) x ragged
lengths x window x query rows per request x forced chunk size x unified
max x soft cap x kernel family x merge place x wave split (tests/sweep_configs.py), each compared
element by element with the fp64 oracle at the KV type's tolerance, and 30
bf16 decodes planned for one CU so that their split partials are row-scaled
fp16 (row_scaled_cases).  Run
with -x: the first failing case stops the run and is named by its index."""
import numpy as np
import pytest

import oracle
from kvs_testlib import compare, poison_invisible, run_library
from sweep_configs import row_scaled_cases, sweep_cases
from workloads import make_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()


def _has_invisible_keys(inp) -> bool:
    s = inp.spec
    rows = np.ones(s.batch, np.int64) if inp.qo_indptr is None else np.diff(inp.qo_indptr)
    return bool(np.any((rows > 0) & (inp.kv_len - rows - s.window + 1 > 0)))


@pytest.mark.parametrize("case", sweep_cases() + row_scaled_cases(), ids=lambda c: c.label())
def test_sweep(case):
    print(f"case sweep {case.label()} lens={case.spec.lengths[1]} q_len={case.spec.q_len}", flush=True)
    inp = make_inputs(case.spec, poison=True)
    if case.poison_invisible and _has_invisible_keys(inp):
        inp = poison_invisible(inp)
    o, lse = run_library(inp, kv_chunk=case.kv_chunk, algo=case.algo, unified_max=case.unified_max,
                         merge_mode=case.merge_mode, wave_split=case.wave_split, num_cus=case.num_cus)
    o_ref, lse_ref = oracle.attention_reference(inp)
    err, rel = compare(o, lse, o_ref, lse_ref, case.spec.kv_dtype)
    print(f"  max|o-o_ref|={err:.2e} lse_rel={rel:.2e}", flush=True)
