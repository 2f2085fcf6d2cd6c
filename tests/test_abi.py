"""The C ABI on the host: symbols, struct layout, validation and planning.

Nothing here launches a kernel; every call returns before any HIP call
(num_cus is given, so planning needs no device query).
"""
import ctypes
import os
import re
import subprocess
import tempfile

import numpy as np
import pytest

import decode_attention_kv_split_amd as kvs
from kvs_testlib import ROOT, ensure_built

HEADER = os.path.join(ROOT, "include", "kvsplit.h")


@pytest.fixture(scope="module")
def lib():
    return ensure_built()


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(kvs_\w+)\s*\(", src, flags=re.M)))


def test_exports_every_declared_function(lib):
    names = _declared_functions()
    assert set(names) >= {"kvs_decode", "kvs_decode_plan", "kvs_decode_workspace_bytes", "kvs_append",
                          "kvs_status_string", "kvs_abi_version"}
    for n in names:
        assert hasattr(lib, n), f"{n} declared in kvsplit.h but not exported"
    out = subprocess.run(["nm", "-D", "--defined-only", kvs.library_path()], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kvs_\w+)", out))
    assert set(names) <= exported


def test_abi_version(lib):
    assert kvs.kvs_abi_version() == kvs.KVS_ABI_VERSION == 12
    assert re.search(r"#define KVS_ABI_VERSION 12\b", open(HEADER).read())
    assert kvs.kvs_status_string(kvs.KVS_ERR_WORKSPACE).startswith("workspace")


def test_struct_layout_matches_header(tmp_path):
    fields = [f[0] for f in kvs.KvsDecodeArgs._fields_]
    pfields = [f[0] for f in kvs.KvsPlanInfo._fields_]
    afields = [f[0] for f in kvs.KvsAppendArgs._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", f'#include "{HEADER}"', "int main(void){"]
    prog.append('printf("%zu\\n", sizeof(kvs_decode_args));')
    prog += [f'printf("%zu\\n", offsetof(kvs_decode_args, {f}));' for f in fields]
    prog.append('printf("%zu\\n", sizeof(kvs_plan_info));')
    prog += [f'printf("%zu\\n", offsetof(kvs_plan_info, {f}));' for f in pfields]
    prog.append('printf("%zu\\n", sizeof(kvs_append_args));')
    prog += [f'printf("%zu\\n", offsetof(kvs_append_args, {f}));' for f in afields]
    prog.append("return 0;}")
    c = tmp_path / "layout.c"
    c.write_text("\n".join(prog))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", str(c), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    want = [ctypes.sizeof(kvs.KvsDecodeArgs)] + [getattr(kvs.KvsDecodeArgs, f).offset for f in fields]
    want += [ctypes.sizeof(kvs.KvsPlanInfo)] + [getattr(kvs.KvsPlanInfo, f).offset for f in pfields]
    want += [ctypes.sizeof(kvs.KvsAppendArgs)] + [getattr(kvs.KvsAppendArgs, f).offset for f in afields]
    assert vals == want


def test_constants_match_header(tmp_path):
    """Every KVS_ constant the header defines (enums and macros) has the same
    value in the binding, and the binding defines no other."""
    names = sorted(set(re.findall(r"\bKVS_[A-Z0-9_]+\b", open(HEADER).read())))
    ours = sorted(n for n in dir(kvs) if n.startswith("KVS_"))
    assert names == ours
    prog = ["#include <stdio.h>", f'#include "{HEADER}"', "int main(void){"]
    prog += [f'printf("%lld\\n", (long long)({n}));' for n in names]
    prog.append("return 0;}")
    c = tmp_path / "consts.c"
    c.write_text("\n".join(prog))
    exe = tmp_path / "consts"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", str(c), "-o", str(exe)], check=True)
    vals = [int(x) for x in subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout.split()]
    assert vals == [int(getattr(kvs, n)) for n in names]


def _args(batch=2, Hq=8, Hk=2, d=128, q=kvs.KVS_BF16, kv=kvs.KVS_BF16, P=16, lens=(100, 3000), window=-1,
          chunk=0, num_pages=1000, algo=0, ptrs=True):
    a = kvs.KvsDecodeArgs()
    a.batch, a.num_qo_heads, a.num_kv_heads, a.head_dim = batch, Hq, Hk, d
    a.q_dtype, a.kv_dtype, a.page_size, a.num_pages = q, kv, P, num_pages
    host = np.asarray(lens, np.int32)
    fake = 0x1000
    if ptrs:
        a.q = a.k = a.v = a.kv_len = a.o = fake
        a.page_indptr = a.page_indices = fake if P else None
        a.k_scale = a.v_scale = fake if kv in (kvs.KVS_FP8_E4M3, kvs.KVS_INT4) else None
    a.kv_len_host = host.ctypes.data
    a.sm_scale = 0.125
    a.window = window
    a.kv_chunk = chunk
    a.algo = algo
    a.num_cus = 256
    return a, host


BAD = [
    (dict(batch=0), kvs.KVS_ERR_INVALID_ARG),
    (dict(Hq=6, Hk=4), kvs.KVS_ERR_INVALID_ARG),
    (dict(Hq=34, Hk=2), kvs.KVS_ERR_UNSUPPORTED),  # group 17 > 16
    (dict(d=96), kvs.KVS_ERR_UNSUPPORTED),
    (dict(q=kvs.KVS_F32, kv=kvs.KVS_BF16), kvs.KVS_ERR_UNSUPPORTED),
    (dict(q=kvs.KVS_BF16, kv=kvs.KVS_F32), kvs.KVS_ERR_UNSUPPORTED),
    (dict(q=7), kvs.KVS_ERR_INVALID_ARG),
    (dict(P=0), kvs.KVS_ERR_INVALID_ARG),  # contiguous with batch 2
    (dict(P=24), kvs.KVS_ERR_UNSUPPORTED),
    (dict(P=-1), kvs.KVS_ERR_INVALID_ARG),
    (dict(window=0), kvs.KVS_ERR_INVALID_ARG),
    (dict(window=-2), kvs.KVS_ERR_INVALID_ARG),
    (dict(chunk=-16), kvs.KVS_ERR_INVALID_ARG),
    (dict(lens=(5, -1)), kvs.KVS_ERR_INVALID_ARG),
    (dict(num_pages=10), kvs.KVS_ERR_INVALID_ARG),  # 3000 tokens need 188 pages of 16
    (dict(algo=9), kvs.KVS_ERR_INVALID_ARG),
    (dict(P=8, algo=kvs.KVS_ALGO_MFMA), kvs.KVS_ERR_UNSUPPORTED),
    (dict(q=kvs.KVS_F32, kv=kvs.KVS_F32, algo=kvs.KVS_ALGO_MFMA), kvs.KVS_ERR_UNSUPPORTED),
    (dict(kv=kvs.KVS_FP8_E4M3, Hq=32, Hk=2, algo=kvs.KVS_ALGO_VALU), kvs.KVS_ERR_UNSUPPORTED),
    (dict(kv=kvs.KVS_INT4, d=64), kvs.KVS_ERR_UNSUPPORTED),                 # INT4 needs head_dim >= 128
    (dict(kv=kvs.KVS_INT4, algo=kvs.KVS_ALGO_VALU), kvs.KVS_ERR_UNSUPPORTED),
    (dict(kv=kvs.KVS_INT4, P=8), kvs.KVS_ERR_UNSUPPORTED),                  # matrix-core kernel: pages >= 16
    (dict(q=kvs.KVS_F32, kv=kvs.KVS_INT4), kvs.KVS_ERR_UNSUPPORTED),
    (dict(kv=4), kvs.KVS_ERR_INVALID_ARG),
    # 2^26 splits of 16 tokens x 32 KV heads: more workgroups than one launch holds
    (dict(batch=1, P=0, Hq=32, Hk=32, lens=(1 << 30,), chunk=16, num_pages=1 << 30), kvs.KVS_ERR_UNSUPPORTED),
    # a contiguous cache holds num_pages tokens
    (dict(batch=1, P=0, lens=(1001,), num_pages=1000), kvs.KVS_ERR_INVALID_ARG),
    (dict(batch=1, P=0, lens=(5,), num_pages=-1), kvs.KVS_ERR_INVALID_ARG),
]


@pytest.mark.parametrize("kw,status", BAD, ids=[str(b[0]) for b in BAD])
def test_validation_before_any_hip_call(lib, kw, status):
    a, keep = _args(**kw)
    assert kvs.kvs_decode(a, 0, 0, 0) == status
    with pytest.raises(kvs.KvsError):
        kvs.kvs_decode_plan(a)
    assert kvs.kvs_decode_workspace_bytes(a) == 0


def test_query_row_checks(lib):
    """Several queries per request: offsets from 0, non-decreasing, at most
    kv_len new tokens each; the matrix-core kernel only."""
    def with_rows(rows, **kw):
        a, keep = _args(**kw)
        qo = np.asarray(rows, np.int32)
        a.qo_indptr, a.qo_indptr_host = 0x2000, qo.ctypes.data
        return a, (keep, qo)
    a, keep = with_rows([0, 3, 10])                     # lens (100, 3000): fine
    assert kvs.kvs_decode_plan(a).col_groups == (7 * 4 + 15) // 16
    assert kvs.kvs_decode_plan(a).col_share == 2   # two groups: the decode kernel runs both
    a, keep = with_rows([0, 12, 20])                    # 12 rows x 4 heads: 3 groups
    assert kvs.kvs_decode_plan(a).col_share == 8        # bf16: the shared-tile kernel, 8 groups a workgroup
    a, keep = with_rows([0, 12, 20], kv=kvs.KVS_FP8_E4M3)
    assert kvs.kvs_decode_plan(a).col_share == 8        # fp8 at head_dim 128: the 32x32 kernel from 3 groups
    a, keep = with_rows([0, 12, 20], kv=kvs.KVS_FP8_E4M3, d=64)
    assert kvs.kvs_decode_plan(a).col_share == 2        # other fp8 shapes: the shared-tile kernel from 5 groups
    a, keep = with_rows([0, 20, 40], kv=kvs.KVS_FP8_E4M3, d=64)
    assert kvs.kvs_decode_plan(a).col_share == 8
    a, keep = with_rows([0, 12, 20], d=256)
    assert kvs.kvs_decode_plan(a).col_share == 4        # head_dim 256: one group per wave
    for rows in ([1, 3, 10], [0, 5, 4], [0, 101, 200]):  # start, decrease, more than kv_len
        a, keep = with_rows(rows)
        assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG, rows
    a, keep = with_rows([0, 3, 10], algo=kvs.KVS_ALGO_VALU)
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_UNSUPPORTED
    a, keep = with_rows([0, 3, 10], algo=kvs.KVS_ALGO_MFMA_PACKED)
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_UNSUPPORTED
    a, keep = _args()
    a.qo_indptr = 0x2000                                # device offsets without the host copy
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG


def test_unified_max_checks(lib):
    a, keep = _args()
    a.use_unified_max, a.unified_max = 1, float("nan")
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG
    a.unified_max = float("inf")
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG
    a.use_unified_max = 2
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG
    a, keep = _args(ptrs=False)
    a.use_unified_max, a.unified_max = 1, 5.0
    assert kvs.kvs_decode_plan(a).items_per_kv_head >= 1


def test_soft_cap_checks(lib):
    for bad in (-1.0, float("nan"), float("inf"), -0.5e-30):
        a, keep = _args()
        a.logits_soft_cap = bad
        assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG, bad
    for algo in (kvs.KVS_ALGO_AUTO, kvs.KVS_ALGO_VALU):
        a, keep = _args(ptrs=False, algo=algo)
        a.logits_soft_cap = 50.0
        assert kvs.kvs_decode_plan(a).items_per_kv_head >= 1


def test_null_pointers_rejected(lib):
    a, keep = _args()
    a.q = None
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG
    a, keep = _args(kv=kvs.KVS_FP8_E4M3)
    a.k_scale = None
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG
    a, keep = _args()
    a.page_indices = None
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG
    # the planner does not need device pointers
    a, keep = _args(ptrs=False)
    assert kvs.kvs_decode_plan(a).items_per_kv_head >= 1


def test_workspace_checks(lib):
    a, keep = _args(lens=(100, 30000), num_pages=4000)
    need = kvs.kvs_decode_workspace_bytes(a)
    assert need > 0
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_WORKSPACE
    assert kvs.kvs_decode(a, 0x10000, need - 1, 0) == kvs.KVS_ERR_WORKSPACE
    assert kvs.kvs_decode(a, 0x10010, need, 0) == kvs.KVS_ERR_WORKSPACE  # not 256-aligned


def _emulate_splits(lens, window, chunk):
    """The device's (request, split) -> token range rule, restated for the test."""
    out = []
    for L in lens:
        lo = max(0, L - window) if window > 0 else 0
        a = lo & ~15
        span = L - a
        n = 1 if span <= 0 else -(-span // chunk)
        out.append([(max(lo, a + s * chunk), min(L, a + (s + 1) * chunk)) for s in range(n)])
    return out


@pytest.mark.parametrize("window", [-1, 1, 7, 512, 5000])
@pytest.mark.parametrize("chunk", [0, 16, 48, 1000, 1 << 20])
def test_plan_tiles_each_request_exactly_once(lib, window, chunk):
    lens = (0, 1, 15, 16, 17, 100, 511, 4097, 30000)
    a, keep = _args(batch=len(lens), lens=lens, window=window, chunk=chunk, num_pages=4000)
    info = kvs.kvs_decode_plan(a)
    assert info.kv_chunk % 16 == 0 and info.kv_chunk > 0
    if chunk:
        assert info.kv_chunk == min(4096, -(-chunk // 16) * 16)
    ranges = _emulate_splits(lens, window, info.kv_chunk)
    assert info.items_per_kv_head == sum(len(r) for r in ranges)
    assert info.max_splits == max(len(r) for r in ranges)
    assert info.needs_merge == (info.max_splits > 1)
    for L, rs in zip(lens, ranges):
        lo = max(0, L - window) if window > 0 else 0
        covered = []
        for t0, t1 in rs:
            covered.extend(range(t0, t1))
        assert covered == list(range(lo, L))
    g = 4
    if info.needs_merge:
        # bf16 decode-kernel partials: fp16 rows, then their LSEs and
        # multipliers, when the launch has more workgroups than CUs; else fp32
        slots = info.items_per_kv_head * 2 * g
        r256 = lambda n: -(-n // 256) * 256
        big = info.items_per_kv_head * 2 > 256
        want = r256(slots * 128 * (2 if big else 4)) + (2 if big else 1) * r256(slots * 4) + r256(len(lens) * 8)
        assert info.workspace_bytes == kvs.KVS_WORKSPACE_COUNTER_BYTES + want  # counters, then the partials
    else:
        assert info.workspace_bytes == 0


@pytest.mark.parametrize("kv,algo,part_bytes,row_scales", [
    (kvs.KVS_BF16, kvs.KVS_ALGO_MFMA, 2, True),    # decode kernel: row-scaled fp16
    (kvs.KVS_BF16, kvs.KVS_ALGO_VALU, 4, False),   # vector kernel: fp32
    (kvs.KVS_FP8_E4M3, kvs.KVS_ALGO_MFMA, 2, False),
    (kvs.KVS_INT4, kvs.KVS_ALGO_MFMA, 2, False),
])
def test_split_partials_size_by_kv_type(lib, kv, algo, part_bytes, row_scales):
    """The split partial outputs are fp16 code averages (V scale applied by
    the merge) for fp8 and INT4 caches; for bf16 caches, fp16 rows with an fp32
    multiplier each from the decode kernel (in launches of more workgroups
    than CUs: 66 here, on 16 CUs), fp32 from the others.  Their LSEs are fp32
    either way."""
    a, keep = _args(kv=kv, lens=(100, 3000, 5000), batch=3, chunk=256, algo=algo)
    a.num_cus = 16
    info = kvs.kvs_decode_plan(a)
    assert info.needs_merge
    g = 4
    slots = info.items_per_kv_head * 2 * g
    r256 = lambda n: -(-n // 256) * 256
    want = r256(slots * 128 * part_bytes) + r256(slots * 4) * (2 if row_scales else 1) + r256(3 * 8)
    assert info.workspace_bytes == kvs.KVS_WORKSPACE_COUNTER_BYTES + want
    fmt = kvs.KVS_PART_F16_ROWS if row_scales else kvs.KVS_PART_F32 if part_bytes == 4 else kvs.KVS_PART_F16_CODES
    assert info.part_format == fmt


@pytest.mark.parametrize("cus,row_scales", [(65, True), (66, False), (256, False)])
def test_bf16_row_scaled_partials_only_past_one_workgroup_per_cu(lib, cus, row_scales):
    """66 decode workgroups (33 items x 2 KV heads): row-scaled fp16 partials
    on fewer CUs, fp32 ones on as many or more."""
    a, keep = _args(lens=(100, 3000, 5000), batch=3, chunk=256)
    a.num_cus = cus
    info = kvs.kvs_decode_plan(a)
    assert info.needs_merge and info.items_per_kv_head == 33
    slots = 33 * 2 * 4
    r256 = lambda n: -(-n // 256) * 256
    want = r256(slots * 128 * (2 if row_scales else 4)) + r256(slots * 4) * (2 if row_scales else 1) + r256(3 * 8)
    assert info.workspace_bytes == kvs.KVS_WORKSPACE_COUNTER_BYTES + want
    assert info.part_format == (kvs.KVS_PART_F16_ROWS if row_scales else kvs.KVS_PART_F32)


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_two_column_groups_store_row_scaled_partials(lib, d):
    """5 to 8 query rows per request at 4 heads per KV head (two groups of 16
    columns, one workgroup: the 32-column kernel at 128, the decode kernel at
    64): row-scaled fp16 partials in a launch past one workgroup per CU."""
    qo = np.array([0, 8, 13, 19], np.int32)
    a, keep = _args(d=d, lens=(1000, 3000, 5000), batch=3, chunk=64)
    a.qo_indptr = 0x1000
    a.qo_indptr_host = qo.ctypes.data
    info = kvs.kvs_decode_plan(a)
    assert info.needs_merge and info.col_groups == 2 and info.col_share == 2
    assert info.part_format == kvs.KVS_PART_F16_ROWS
    slots = info.items_per_kv_head * 2 * 32
    r256 = lambda n: -(-n // 256) * 256
    want = r256(slots * d * 2) + 2 * r256(slots * 4) + r256(3 * 8)
    assert info.workspace_bytes == kvs.KVS_WORKSPACE_COUNTER_BYTES + want


@pytest.mark.parametrize("d,row_scales", [(64, False), (128, True), (256, True)])
def test_bf16_partials_of_the_multi_row_kernels(lib, d, row_scales):
    """bf16 caches with enough query rows per request for the shared-tile or
    32x32 kernels (col_share >= 4): row-scaled fp16 partials from the 32x32
    prefill kernel (head_dim 128: a row is one wave's; 256: a wave pair's);
    fp32 ones from the shared-tile kernel (head_dim 64)."""
    qo = np.array([0, 40, 80, 120], np.int32)
    a, keep = _args(d=d, lens=(1000, 3000, 5000), batch=3, chunk=256)
    a.qo_indptr = 0x1000
    a.qo_indptr_host = qo.ctypes.data
    a.num_cus = 16  # 144 workgroups: past one per CU
    info = kvs.kvs_decode_plan(a)
    assert info.needs_merge and info.col_share >= 4
    cols = 16 * -(-40 * 4 // 16)  # (query row, head) columns per KV head: 10 groups of 16
    slots = info.items_per_kv_head * 2 * cols
    r256 = lambda n: -(-n // 256) * 256
    want = r256(slots * d * (2 if row_scales else 4)) + r256(slots * 4) * (2 if row_scales else 1) + r256(3 * 8)
    assert info.workspace_bytes == kvs.KVS_WORKSPACE_COUNTER_BYTES + want
    assert info.part_format == (kvs.KVS_PART_F16_ROWS if row_scales else kvs.KVS_PART_F32)


def test_plan_heuristic_fills_the_gpu_at_batch_one(lib):
    a, keep = _args(batch=1, Hq=32, Hk=32, P=0, lens=(32768,), num_pages=32768)
    cus = a.num_cus
    for split, packs in (("tiles", 1), ("heads", 4), ("auto", 4)):
        a.wave_split = {"auto": 0, "heads": 1, "tiles": 2}[split]
        a.num_cus = cus
        info = kvs.kvs_decode_plan(a)
        assert info.wave_packs == packs
        # at least one workgroup per CU, each with the same work either way
        assert info.items_per_kv_head * 32 // packs >= 256
        assert info.kv_chunk * packs >= 512
        assert info.kv_chunk % 16 == 0 and info.kv_chunk <= (1024 if packs == 4 else 4096)
        assert info.algo == kvs.KVS_ALGO_MFMA
        a.num_cus = 64
        assert kvs.kvs_decode_plan(a).kv_chunk >= info.kv_chunk
        # deterministic
        assert kvs.kvs_decode_plan(a).kv_chunk == kvs.kvs_decode_plan(a).kv_chunk


def test_algo_resolution(lib):
    a, keep = _args(q=kvs.KVS_F32, kv=kvs.KVS_F32, Hq=8, Hk=8, d=64, batch=1, P=0, lens=(512,), num_pages=512)
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_VALU
    a, keep = _args(P=8)
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_VALU
    a, keep = _args(kv=kvs.KVS_FP8_E4M3)
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA
    a.algo = kvs.KVS_ALGO_MFMA_PACKED
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA_PACKED
    a, keep = _args(q=kvs.KVS_F32, kv=kvs.KVS_F32, Hq=8, Hk=8, d=64, batch=1, P=0, lens=(512,), num_pages=512,
                    algo=kvs.KVS_ALGO_MFMA_PACKED)
    with pytest.raises(kvs.KvsError):
        kvs.kvs_decode_plan(a)


# ------------------------------------------------------------------ kvs_append

def _append_args(batch=2, Hq=8, Hk=2, d=128, q=kvs.KVS_BF16, kv=kvs.KVS_BF16, P=16, num_pages=100,
                 eps=1e-6, theta=1e4, interleave=0):
    a = kvs.KvsAppendArgs()
    a.batch, a.num_qo_heads, a.num_kv_heads, a.head_dim = batch, Hq, Hk, d
    a.q_dtype, a.kv_dtype, a.page_size, a.num_pages = q, kv, P, num_pages
    fake = 0x1000
    a.q_in = a.k_in = a.v_in = a.q_out = a.k_cache = a.v_cache = a.kv_len = fake
    a.page_indptr = a.page_indices = fake if P else None
    a.k_scale = a.v_scale = fake if kv in (kvs.KVS_FP8_E4M3, kvs.KVS_INT4) else None
    a.norm_eps, a.rope_theta, a.rope_interleave = eps, theta, interleave
    return a


BAD_APPEND = [
    (dict(batch=0), kvs.KVS_ERR_INVALID_ARG),
    (dict(Hq=6, Hk=4), kvs.KVS_ERR_INVALID_ARG),
    (dict(d=96), kvs.KVS_ERR_UNSUPPORTED),
    (dict(q=kvs.KVS_F32, kv=kvs.KVS_BF16), kvs.KVS_ERR_UNSUPPORTED),
    (dict(q=5), kvs.KVS_ERR_INVALID_ARG),
    (dict(kv=kvs.KVS_INT4, d=64), kvs.KVS_ERR_UNSUPPORTED),     # INT4 caches: head_dim 128 or 256
    (dict(q=kvs.KVS_F32, kv=kvs.KVS_INT4), kvs.KVS_ERR_UNSUPPORTED),
    (dict(P=0), kvs.KVS_ERR_INVALID_ARG),          # contiguous with batch 2
    (dict(P=24), kvs.KVS_ERR_UNSUPPORTED),
    (dict(P=-16), kvs.KVS_ERR_INVALID_ARG),
    (dict(num_pages=0), kvs.KVS_ERR_INVALID_ARG),
    (dict(eps=-1.0), kvs.KVS_ERR_INVALID_ARG),
    (dict(eps=float("nan")), kvs.KVS_ERR_INVALID_ARG),
    (dict(theta=-1.0), kvs.KVS_ERR_INVALID_ARG),
    (dict(theta=float("inf")), kvs.KVS_ERR_INVALID_ARG),
    (dict(interleave=2), kvs.KVS_ERR_INVALID_ARG),
    (dict(batch=1 << 22, Hq=32, Hk=8), kvs.KVS_ERR_UNSUPPORTED),  # 2^22 * 40 rows exceed one launch
]


@pytest.mark.parametrize("kw,status", BAD_APPEND, ids=[str(b[0]) for b in BAD_APPEND])
def test_append_validation_before_any_hip_call(lib, kw, status):
    assert kvs.kvs_append(_append_args(**kw), 0) == status


def test_append_token_row_checks(lib):
    """A packed ragged batch: both row arrays or neither, offsets from 0,
    never decreasing; INT4 caches accepted at head_dim 128 / 256."""
    def with_rows(rows, dev=True, **kw):
        a = _append_args(**kw)
        qo = np.asarray(rows, np.int32)
        a.qo_indptr, a.qo_indptr_host = (0x2000 if dev else None), qo.ctypes.data
        return a, qo
    for rows, dev, want in (([0, 3, 5], True, None), ([0, 0, 0], True, None), ([1, 3, 5], True, kvs.KVS_ERR_INVALID_ARG),
                            ([0, 4, 2], True, kvs.KVS_ERR_INVALID_ARG), ([0, 3, 5], False, kvs.KVS_ERR_INVALID_ARG)):
        a, keep = with_rows(rows, dev)
        if want is not None:
            assert kvs.kvs_append(a, 0) == want, rows
    a = _append_args()
    a.qo_indptr = 0x2000  # device array without its host copy
    assert kvs.kvs_append(a, 0) == kvs.KVS_ERR_INVALID_ARG
    a, keep = with_rows([0, 1 << 22, 1 << 23], Hq=32, Hk=8)  # 2^23 token rows x 40 head rows: too many
    assert kvs.kvs_append(a, 0) == kvs.KVS_ERR_UNSUPPORTED
    a = _append_args(kv=kvs.KVS_INT4)
    a.k_scale = None
    assert kvs.kvs_append(a, 0) == kvs.KVS_ERR_INVALID_ARG


def test_append_null_pointers_rejected(lib):
    for field in ("q_in", "k_in", "v_in", "q_out", "k_cache", "v_cache", "kv_len", "page_indptr", "page_indices"):
        a = _append_args()
        setattr(a, field, None)
        assert kvs.kvs_append(a, 0) == kvs.KVS_ERR_INVALID_ARG, field
    a = _append_args(kv=kvs.KVS_FP8_E4M3)
    a.v_scale = None
    assert kvs.kvs_append(a, 0) == kvs.KVS_ERR_INVALID_ARG


def test_int4_packs_two_heads_when_it_can(lib):
    """AUTO resolves INT4 head_dim 128 with one query per request to the
    two-heads-per-workgroup kernel (a 64-byte head row is half a line)."""
    a, keep = _args(kv=kvs.KVS_INT4, ptrs=False)                 # 8 query / 2 KV heads
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA_PACKED
    a, keep = _args(kv=kvs.KVS_INT4, Hq=32, Hk=2, ptrs=False)    # group 16: 32 columns do not fit
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA
    a, keep = _args(kv=kvs.KVS_INT4, Hq=9, Hk=3, ptrs=False)     # odd KV head count
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA
    a, keep = _args(kv=kvs.KVS_INT4, d=256, ptrs=False)          # 128-byte rows: whole lines already
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA
    a, keep = _args(kv=kvs.KVS_INT4, algo=kvs.KVS_ALGO_MFMA, ptrs=False)  # asked for one head
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA
    a, keep = _args(kv=kvs.KVS_FP8_E4M3, ptrs=False)             # fp8 stays unpacked by default
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA


# ----------------------------------------------------------------------------
# the Python binding rejects buffers the kernels would overrun, before it
# looks at where the tensors live (so these checks run on the CPU)
# ----------------------------------------------------------------------------

def _torch_case(L=40, cap=40, paged=False):
    import torch

    q = torch.zeros(1, 8, 64, dtype=torch.bfloat16)
    if paged:
        k = torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16)
        extra = dict(page_indptr=torch.tensor([0, 3], dtype=torch.int32),
                     page_indices=torch.tensor([0, 1, 2], dtype=torch.int32))
    else:
        k = torch.zeros(cap, 2, 64, dtype=torch.bfloat16)
        extra = {}
    return q, k, k.clone(), torch.tensor([L], dtype=torch.int32), extra


@pytest.mark.parametrize("bad", ["out_shape", "out_dtype", "lse_shape", "lse_dtype", "kv_len_past_cache"])
def test_binding_rejects_unsafe_buffers(bad):
    import torch

    q, k, v, kv_len, extra = _torch_case(L=41 if bad == "kv_len_past_cache" else 40)
    kw = {}
    if bad == "out_shape":
        kw["out"] = torch.empty(1, 8, 32, dtype=torch.bfloat16)
    elif bad == "out_dtype":
        kw["out"] = torch.empty(1, 8, 64, dtype=torch.float32)
    elif bad == "lse_shape":
        kw["lse"] = torch.empty(1, 4, dtype=torch.float32)
    elif bad == "lse_dtype":
        kw["lse"] = torch.empty(1, 8, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must|lse must|exceeds the rows"):
        kvs.make_args(q, k, v, kv_len, kv_len_host=[int(kv_len[0])], **kw, **extra)


def test_binding_passes_contiguous_capacity():
    """A well-formed case gets past every shape check (it then stops at the
    device check, since these tensors are on the CPU)."""
    q, k, v, kv_len, extra = _torch_case(L=40, cap=64)
    with pytest.raises(ValueError, match="must be on"):
        kvs.make_args(q, k, v, kv_len, kv_len_host=[40])


def test_noalloc_rejects_oversized_calls_before_any_hip_call(lib):
    """kvs_decode_noalloc validates like kvs_decode, then refuses a call whose
    split partials would not fit its fixed device array."""
    a, keep = _args(batch=1, Hq=32, Hk=32, P=0, lens=(1 << 20,), chunk=16, num_pages=1 << 20)
    assert kvs.kvs_decode_workspace_bytes(a) > kvs.KVS_NOALLOC_SCRATCH_BYTES
    assert kvs.kvs_decode_noalloc(a, 0) == kvs.KVS_ERR_TOO_LARGE
    assert "KVS_NOALLOC_SCRATCH_BYTES" in kvs.kvs_status_string(kvs.KVS_ERR_TOO_LARGE)
    a, keep = _args(window=0)
    assert kvs.kvs_decode_noalloc(a, 0) == kvs.KVS_ERR_INVALID_ARG
    assert re.search(r"#define KVS_NOALLOC_SCRATCH_BYTES \(\(size_t\)32 << 20\)", open(HEADER).read())
    assert kvs.KVS_NOALLOC_SCRATCH_BYTES == 32 << 20


def test_merge_runs_in_the_partial_kernel_when_the_plan_allows(lib):
    """Asked for (merge_mode IN_PARTIAL), the partial kernel merges for
    host-planned work lists whose counters fit; a second merge kernel runs
    otherwise."""
    real = globals()["_args"]

    def _args(**kw):  # noqa: F811 (this test asks for the in-kernel merge)
        a, keep = real(**kw)
        a.merge_mode = kvs.KVS_MERGE_IN_PARTIAL
        return a, keep

    a, keep = _args(ptrs=False)                                    # 2 requests, split
    info = kvs.kvs_decode_plan(a)
    assert info.needs_merge and info.merge_in_partial == 1
    assert info.workspace_bytes >= kvs.KVS_WORKSPACE_COUNTER_BYTES
    a, keep = _args(ptrs=False, lens=(10, 20))                     # nothing to merge: no workspace
    info = kvs.kvs_decode_plan(a)
    assert not info.needs_merge and info.merge_in_partial == 0 and info.workspace_bytes == 0
    a, keep = _args(ptrs=False, batch=300, lens=(700,) * 300, num_pages=20000, chunk=64)  # device work list
    assert kvs.kvs_decode_plan(a).merge_in_partial == 0
    a, keep = _args(ptrs=False, batch=1, lens=(8192,), chunk=16, num_pages=600)  # 512 splits > 256
    assert kvs.kvs_decode_plan(a).merge_in_partial == 0
    a, keep = _args(ptrs=False, batch=200, lens=(650,) * 200, chunk=128, num_pages=9000)  # 1200 items: inline
    assert kvs.kvs_decode_plan(a).items_per_kv_head == 1200 and kvs.kvs_decode_plan(a).merge_in_partial == 1
    a, keep = _args(ptrs=False, batch=250, lens=(1000,) * 250, chunk=128, num_pages=16000)  # 2000 items > 1344
    assert kvs.kvs_decode_plan(a).merge_in_partial == 0
    # 200 requests x 128 KV heads = 25,600 counters > 16,384
    a, keep = _args(ptrs=False, batch=200, Hq=128, Hk=128, d=64, lens=(32,) * 200, chunk=16, num_pages=1000)
    info = kvs.kvs_decode_plan(a)
    assert info.needs_merge and info.merge_in_partial == 0
    # the INT4 head_dim-256 shared-tile kernel leaves its merge to the merge kernel
    a, keep = _args(ptrs=False, kv=kvs.KVS_INT4, d=256, lens=(700, 1500), chunk=256)
    rows = np.array([0, 40, 80], np.int32)
    a.qo_indptr_host = rows.ctypes.data
    info = kvs.kvs_decode_plan(a)
    assert info.col_share >= 4 and info.needs_merge and info.merge_in_partial == 0
    a.kv_dtype = kvs.KVS_BF16                                      # the bf16 one merges itself
    info = kvs.kvs_decode_plan(a)
    assert info.col_share >= 4 and info.merge_in_partial == 1


def test_merge_mode_auto_and_kernel(lib):
    """AUTO merges inside the partial kernel only for launches of at most one
    workgroup per CU (there a second launch costs more than the merge);
    KERNEL always takes the merge kernel; other values are rejected."""
    a, keep = _args(ptrs=False, batch=1, P=0, Hq=8, Hk=8, d=64, q=kvs.KVS_F32, kv=kvs.KVS_F32,
                    lens=(512,), num_pages=512)                    # 8 chunks x 8 heads = 64 workgroups
    assert kvs.kvs_decode_plan(a).merge_in_partial == 1
    a.merge_mode = kvs.KVS_MERGE_KERNEL
    assert kvs.kvs_decode_plan(a).merge_in_partial == 0
    a, keep = _args(ptrs=False, batch=1, P=0, Hq=32, Hk=32, lens=(32768,), num_pages=32768)  # 2048 workgroups
    assert kvs.kvs_decode_plan(a).merge_in_partial == 0
    a.merge_mode = kvs.KVS_MERGE_IN_PARTIAL
    assert kvs.kvs_decode_plan(a).merge_in_partial == 1
    a.merge_mode = 3
    assert kvs.kvs_decode(a, 0, 0, 0) == kvs.KVS_ERR_INVALID_ARG


def _plan_status(a):
    try:
        kvs.kvs_decode_plan(a)
    except kvs.KvsError as e:
        return e.status
    return kvs.KVS_OK


def test_wave_split_choice_and_validation(lib):
    """One KV-head pack per wave when asked for (HEADS) where the packs come
    in fours with one query row per request, and automatically where it can
    keep the tiles split's chunks (at most 1024 keys) with a workgroup per
    CU; the tiles split otherwise.  HEADS asked for where it does not apply
    is unsupported, unknown values are invalid."""
    # GQA paged decode, 8 KV heads: two workgroups of four packs per chunk
    a, keep = _args(ptrs=False, batch=3, Hq=32, Hk=8, lens=(100, 4000, 18000), num_pages=2000)
    a.wave_split = kvs.KVS_WAVES_TILES
    tiles = kvs.kvs_decode_plan(a)
    assert tiles.wave_packs == 1 and tiles.kv_chunk <= 1024
    a.wave_split = kvs.KVS_WAVES_AUTO                      # same chunks, 348 workgroups: heads
    info = kvs.kvs_decode_plan(a)
    assert info.wave_packs == 4 and info.kv_chunk == tiles.kv_chunk
    assert info.items_per_kv_head == tiles.items_per_kv_head and info.workspace_bytes == tiles.workspace_bytes
    a.num_cus = 1024                                       # fewer workgroups than CUs: tiles
    assert kvs.kvs_decode_plan(a).wave_packs == 1
    a.num_cus = 256
    # a batch whose tiles chunks exceed 1024 keys keeps the tiles split
    big, keep2 = _args(ptrs=False, batch=64, Hq=32, Hk=8, lens=tuple(range(512, 16384, 248))[:64], num_pages=70000)
    info = kvs.kvs_decode_plan(big)
    assert info.kv_chunk > 1024 and info.wave_packs == 1
    a.wave_split = kvs.KVS_WAVES_HEADS
    info = kvs.kvs_decode_plan(a)
    assert info.wave_packs == 4 and info.kv_chunk % 16 == 0 and info.kv_chunk <= 1024
    a.kv_chunk = 4096                                      # capped at 64 tiles per wave
    assert kvs.kvs_decode_plan(a).kv_chunk == 1024
    a.wave_split = kvs.KVS_WAVES_TILES
    info = kvs.kvs_decode_plan(a)
    assert info.wave_packs == 1 and info.kv_chunk == 4096
    a.wave_split = 3
    assert _plan_status(a) == kvs.KVS_ERR_INVALID_ARG
    # INT4 head_dim 128: two heads per pack, 8 heads -> 4 packs, one workgroup
    a, keep = _args(ptrs=False, batch=2, Hq=64, Hk=8, kv=kvs.KVS_INT4, lens=(500, 3000))
    a.wave_split = kvs.KVS_WAVES_HEADS
    info = kvs.kvs_decode_plan(a)
    assert info.algo == kvs.KVS_ALGO_MFMA_PACKED and info.wave_packs == 4
    # not in fours: one KV head; 6 KV heads
    for Hk in (1, 2, 6):
        a, keep = _args(ptrs=False, batch=2, Hq=6 * Hk, Hk=Hk, lens=(500, 3000))
        assert kvs.kvs_decode_plan(a).wave_packs == 1
        a.wave_split = kvs.KVS_WAVES_HEADS
        assert _plan_status(a) == kvs.KVS_ERR_UNSUPPORTED
    # several query rows per request, and the vector kernel: tiles only
    a, keep = _args(ptrs=False, batch=2, Hq=32, Hk=8, lens=(500, 3000))
    rows = np.array([0, 2, 5], np.int32)
    a.qo_indptr_host = rows.ctypes.data
    assert kvs.kvs_decode_plan(a).wave_packs == 1
    a.wave_split = kvs.KVS_WAVES_HEADS
    assert _plan_status(a) == kvs.KVS_ERR_UNSUPPORTED
    a, keep = _args(ptrs=False, batch=2, Hq=32, Hk=8, q=kvs.KVS_F32, kv=kvs.KVS_F32, lens=(500, 3000))
    info = kvs.kvs_decode_plan(a)
    assert info.algo == kvs.KVS_ALGO_VALU and info.wave_packs == 1
    a.wave_split = kvs.KVS_WAVES_HEADS
    assert _plan_status(a) == kvs.KVS_ERR_UNSUPPORTED


def test_q_and_o_must_be_16_byte_aligned(lib):
    """Rows of q and o move in 16-byte pieces: a misaligned pointer is an
    invalid argument, reported before any launch."""
    for field in ("q", "o"):
        a, keep = _args()
        setattr(a, field, 0x1008)
        ws = (ctypes.c_uint8 * 256)()
        assert kvs.kvs_decode(a, ctypes.addressof(ws), 0, None) == kvs.KVS_ERR_INVALID_ARG
