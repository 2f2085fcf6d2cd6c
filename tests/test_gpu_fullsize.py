"""The three large workloads at full size, in the launch configuration the
benchmark times (heuristic split count, matrix-core kernel), checked on
sampled (request, head) outputs that the oracle computes one by one."""
import numpy as np
import pytest

import oracle
from kvs_testlib import compare, run_library, to_torch
from workloads import CONFIGS, make_inputs

pytestmark = pytest.mark.gpu


def _sampled(name, n_req):
    import torch

    print(f"case {name} full size: drawing inputs", flush=True)
    inp = make_inputs(CONFIGS[name])
    t = to_torch(inp)
    o, lse = run_library(inp, tensors=t)
    del t
    torch.cuda.empty_cache()
    s = inp.spec
    L = inp.kv_len
    reqs = sorted({int(np.argmin(L)), int(np.argmax(L))} |
                  set(np.random.default_rng(0).choice(s.batch, size=min(n_req, s.batch), replace=False).tolist()))
    picks = [(b, h) for b in reqs for h in range(s.num_qo_heads)]
    print(f"case {name}: oracle on requests {reqs}", flush=True)
    ref = oracle.decode_reference_sampled(inp, picks)
    o_ref = np.stack([r[0] for r in ref])
    lse_ref = np.array([r[1] for r in ref])
    idx = tuple(np.array(picks).T)
    compare(o[idx], lse[idx], o_ref, lse_ref, s.kv_dtype)
    assert np.all(np.isfinite(o))


def test_c3_full():
    _sampled("c3_llama2_7b_32k", 1)


def test_c4_full_sampled():
    _sampled("c4_paged_bf16_b64", 3)


def test_c5_full_sampled():
    _sampled("c5_paged_fp8_b128", 3)
