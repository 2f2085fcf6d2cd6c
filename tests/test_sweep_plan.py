"""Every case of the randomized parity sweep is one the library accepts:
planned through the C ABI on the host (no kernel launch, num_cus given)."""
import numpy as np
import pytest

import decode_attention_kv_split_amd as kvs
from kvs_testlib import ensure_built
from sweep_configs import row_scaled_cases, sweep_cases
from workloads import make_inputs

_DT = {"f32": kvs.KVS_F32, "bf16": kvs.KVS_BF16, "fp8": kvs.KVS_FP8_E4M3, "int4": kvs.KVS_INT4}


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def test_sweep_is_seeded_and_varied():
    a, b = sweep_cases(), sweep_cases()
    assert [c.label() for c in a] == [c.label() for c in b]
    kinds = {(c.spec.kv_dtype, c.multi) for c in a}
    assert {("f32", False), ("bf16", True), ("fp8", True), ("int4", True), ("int4", False)} <= kinds
    assert sum(c.spec.window > 0 for c in a) > 30 and sum(c.spec.soft_cap > 0 for c in a) > 20
    assert sum(c.unified_max is not None for c in a) > 10 and sum(c.kv_chunk > 0 for c in a) > 50
    assert {c.algo for c in a} == {"auto", "valu", "mfma_packed"}
    assert {c.merge_mode for c in a} == {"auto", "in_partial", "kernel"}


def _plan(case):
    """kvs_decode_plan of a sweep case (host only; fake device pointers)."""
    s = case.spec
    inp = make_inputs(s)
    a = kvs.KvsDecodeArgs()
    a.batch, a.num_qo_heads, a.num_kv_heads, a.head_dim = s.batch, s.num_qo_heads, s.num_kv_heads, s.head_dim
    a.q_dtype, a.kv_dtype, a.page_size = _DT[s.q_dtype], _DT[s.kv_dtype], s.page_size
    a.num_pages = inp.num_pages if s.page_size else int(inp.k.shape[0])
    fake = 0x1000
    a.q = a.k = a.v = a.kv_len = a.o = fake
    if s.page_size:
        a.page_indptr = a.page_indices = fake
    if s.kv_dtype in ("fp8", "int4"):
        a.k_scale = a.v_scale = fake
    host = np.ascontiguousarray(inp.kv_len, np.int32)
    a.kv_len_host = host.ctypes.data
    qo = None
    if inp.qo_indptr is not None:
        qo = np.ascontiguousarray(inp.qo_indptr, np.int32)
        a.qo_indptr, a.qo_indptr_host = fake, qo.ctypes.data
    a.sm_scale = s.sm_scale
    a.window = s.window
    a.kv_chunk = case.kv_chunk
    a.algo = {"auto": 0, "valu": 1, "mfma": 2, "mfma_packed": 3}[case.algo]
    a.num_cus = case.num_cus or 256
    if case.unified_max is not None:
        a.use_unified_max, a.unified_max = 1, case.unified_max
    a.logits_soft_cap = s.soft_cap
    a.merge_mode = {"auto": 0, "in_partial": 1, "kernel": 2}[case.merge_mode]
    a.wave_split = {"auto": 0, "heads": 1, "tiles": 2}[case.wave_split]
    return kvs.kvs_decode_plan(a)  # raises on any status but KVS_OK


@pytest.mark.parametrize("case", sweep_cases(), ids=lambda c: c.label())
def test_sweep_case_plans(lib, case):
    info = _plan(case)
    assert info.wave_packs in ((4,) if case.wave_split == "heads" else (1, 4))
    assert info.items_per_kv_head >= case.spec.batch


def test_sweep_covers_every_partial_format(lib):
    """Cases whose requests split: bf16 ones with fp32 partials (vector kernel,
    several rows, small launches), fp8 / INT4 ones with fp16 code averages,
    fp32 ones in fp32; the row-scaled set with row-scaled fp16 partials."""
    seen = {}
    for case in sweep_cases():
        info = _plan(case)
        if info.needs_merge:
            key = (case.spec.kv_dtype, info.part_format)
            seen[key] = seen.get(key, 0) + 1
    assert seen.get(("bf16", kvs.KVS_PART_F32), 0) >= 5, seen
    assert seen.get(("fp8", kvs.KVS_PART_F16_CODES), 0) >= 10, seen
    assert seen.get(("int4", kvs.KVS_PART_F16_CODES), 0) >= 10, seen
    assert seen.get(("f32", kvs.KVS_PART_F32), 0) >= 3, seen
    rows = [_plan(c) for c in row_scaled_cases()]
    split = [i for i in rows if i.needs_merge]
    assert len(split) >= 20 and all(i.part_format == kvs.KVS_PART_F16_ROWS for i in split)


@pytest.mark.parametrize("case", row_scaled_cases(), ids=lambda c: c.label())
def test_row_scaled_case_plans(lib, case):
    info = _plan(case)
    assert info.part_format == (kvs.KVS_PART_F16_ROWS if info.needs_merge else kvs.KVS_PART_F32)
