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
    assert kvs.kvs_abi_version() == kvs.KVS_ABI_VERSION == 7
    assert re.search(r"#define KVS_ABI_VERSION 7\b", open(HEADER).read())
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
    (dict(batch=1, P=0, Hq=32, Hk=32, lens=(1 << 30,), chunk=16), kvs.KVS_ERR_UNSUPPORTED),
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
        slots = info.items_per_kv_head * 2 * g
        want = (-(-slots * 128 * 4 // 256) * 256) + (-(-slots * 4 // 256) * 256) + (-(-len(lens) * 8 // 256) * 256)
        assert info.workspace_bytes == want
    else:
        assert info.workspace_bytes == 0


def test_plan_heuristic_fills_the_gpu_at_batch_one(lib):
    a, keep = _args(batch=1, Hq=32, Hk=32, P=0, lens=(32768,), num_pages=0)
    info = kvs.kvs_decode_plan(a)
    assert info.items_per_kv_head * 32 >= 256  # at least one chunk per CU
    assert info.kv_chunk >= 512
    assert info.algo == kvs.KVS_ALGO_MFMA
    a.num_cus = 64
    assert kvs.kvs_decode_plan(a).kv_chunk >= info.kv_chunk
    # deterministic
    assert kvs.kvs_decode_plan(a).kv_chunk == kvs.kvs_decode_plan(a).kv_chunk


def test_algo_resolution(lib):
    a, keep = _args(q=kvs.KVS_F32, kv=kvs.KVS_F32, Hq=8, Hk=8, d=64, batch=1, P=0, lens=(512,), num_pages=0)
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_VALU
    a, keep = _args(P=8)
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_VALU
    a, keep = _args(kv=kvs.KVS_FP8_E4M3)
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA
    a.algo = kvs.KVS_ALGO_MFMA_PACKED
    assert kvs.kvs_decode_plan(a).algo == kvs.KVS_ALGO_MFMA_PACKED
    a, keep = _args(q=kvs.KVS_F32, kv=kvs.KVS_F32, Hq=8, Hk=8, d=64, batch=1, P=0, lens=(512,), num_pages=0,
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
    a.k_scale = a.v_scale = fake if kv == kvs.KVS_FP8_E4M3 else None
    a.norm_eps, a.rope_theta, a.rope_interleave = eps, theta, interleave
    return a


BAD_APPEND = [
    (dict(batch=0), kvs.KVS_ERR_INVALID_ARG),
    (dict(Hq=6, Hk=4), kvs.KVS_ERR_INVALID_ARG),
    (dict(d=96), kvs.KVS_ERR_UNSUPPORTED),
    (dict(q=kvs.KVS_F32, kv=kvs.KVS_BF16), kvs.KVS_ERR_UNSUPPORTED),
    (dict(q=5), kvs.KVS_ERR_INVALID_ARG),
    (dict(kv=kvs.KVS_INT4), kvs.KVS_ERR_UNSUPPORTED),           # the step does not write INT4 caches
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
