"""HIP path against the fp64 oracle on the GPU, element by element.

Tolerances (max |o - o_ref|): 1e-5 for fp32 KV, 2e-2 for bf16 KV, 6e-2 for
fp8 KV; lse within 1e-3 relative (|dlse| <= 1e-3 * max(1, |lse_ref|)).
"""
import dataclasses
import math

import numpy as np
import pytest

import oracle
from kvs_testlib import O_TOL, compare, run_library, to_torch
from workloads import CONFIGS, DecodeSpec, make_inputs, small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()  # raises if libkvsplit.so is not built


def _check(inp, **kw):
    o, lse = run_library(inp, **kw)
    o_ref, lse_ref = oracle.decode_reference(inp)
    return compare(o, lse, o_ref, lse_ref, inp.spec.kv_dtype)


# ---------------------------------------------------------------- the five workloads

def test_c1_mha_f32_full():
    print("case c1 full", flush=True)
    _check(make_inputs(CONFIGS["c1_mha_f32"]))


@pytest.mark.parametrize("name", ["c2_gemma3_1b", "c2_gemma3_1b_w512"])
def test_c2_gemma_full(name):
    print(f"case {name} full", flush=True)
    _check(make_inputs(CONFIGS[name]))


@pytest.mark.parametrize("L", [1, 17, 1000, 4096])
def test_c3_llama_shape_small(L):
    print(f"case c3 L={L}", flush=True)
    spec = small_variant("c3_llama2_7b_32k", lengths=("fixed", L))
    _check(make_inputs(spec))


def test_c4_paged_bf16_small_ragged():
    print("case c4 small ragged", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=7, lengths=("list", [1, 16, 17, 333, 2048, 5000, 40]))
    _check(make_inputs(spec, poison=True))


def test_c5_paged_fp8_small_ragged():
    print("case c5 small ragged", flush=True)
    spec = small_variant("c5_paged_fp8_b128", batch=6, lengths=("list", [128, 1, 700, 3000, 16, 4111]))
    _check(make_inputs(spec, poison=True))


# ---------------------------------------------------------------- split invariance

@pytest.mark.parametrize("algo", ["mfma", "valu"])
@pytest.mark.parametrize("chunk", [0, 16, 32, 48, 64, 1024, 1 << 20])
def test_forced_chunks_bf16(algo, chunk):
    print(f"case chunks bf16 algo={algo} chunk={chunk}", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=4, lengths=("list", [5, 300, 1500, 2049]))
    _check(make_inputs(spec, poison=True), kv_chunk=chunk, algo=algo)


@pytest.mark.parametrize("algo", ["mfma", "valu"])
@pytest.mark.parametrize("chunk", [0, 16, 48, 1024])
def test_forced_chunks_fp8(algo, chunk):
    print(f"case chunks fp8 algo={algo} chunk={chunk}", flush=True)
    spec = small_variant("c5_paged_fp8_b128", batch=3, lengths=("list", [200, 1000, 1777]))
    _check(make_inputs(spec, poison=True), kv_chunk=chunk, algo=algo)


@pytest.mark.parametrize("chunk", [16, 64, 0])
def test_forced_chunks_f32(chunk):
    print(f"case chunks f32 chunk={chunk}", flush=True)
    spec = dataclasses.replace(CONFIGS["c1_mha_f32"], lengths=("fixed", 777))
    _check(make_inputs(spec), kv_chunk=chunk)


# ---------------------------------------------------------------- shapes

@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("g", [1, 2, 4, 8, 16])
def test_head_dims_and_groups(kv, d, g):
    print(f"case shape kv={kv} d={d} g={g}", flush=True)
    Hk = 2
    spec = DecodeSpec("shape", 2, Hk * g, Hk, d, 16, kv, "f32" if kv == "f32" else "bf16", 1 / math.sqrt(d),
                      lengths=("list", [77, 600]), seed=11 + d + g)
    if kv == "fp8" and g == 16:
        _check(make_inputs(spec), algo="mfma")  # the vector kernel takes groups up to 8 for fp8
    else:
        _check(make_inputs(spec))


@pytest.mark.parametrize("P", [1, 2, 8, 16, 32, 64])
def test_page_sizes(P):
    print(f"case page size {P}", flush=True)
    spec = DecodeSpec("pages", 3, 8, 2, 128, P, "bf16", "bf16", 0.1, lengths=("list", [1, 90, 1000]), seed=P)
    _check(make_inputs(spec, poison=True))


@pytest.mark.parametrize("W", [1, 15, 16, 17, 100, 512, 4096])
def test_sliding_window(W):
    print(f"case window {W}", flush=True)
    spec = DecodeSpec("win", 3, 8, 2, 128, 16, "bf16", "bf16", 0.1, window=W,
                      lengths=("list", [3, 600, 2500]), seed=W)
    _check(make_inputs(spec, poison=True))
    spec8 = dataclasses.replace(spec, kv_dtype="fp8")
    _check(make_inputs(spec8, poison=True))


def test_kv_len_edge_cases():
    print("case kv_len edges", flush=True)
    lens = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 4095, 4096, 4097]
    spec = DecodeSpec("edges", len(lens), 8, 2, 128, 16, "bf16", "bf16", 0.1, lengths=("list", lens), seed=5)
    inp = make_inputs(spec, poison=True)
    for chunk in (0, 16, 64):
        o, lse = run_library(inp, kv_chunk=chunk)
        o_ref, lse_ref = oracle.decode_reference(inp)
        compare(o, lse, o_ref, lse_ref, "bf16")
        assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))


@pytest.mark.parametrize("codes", ["all_finite", "subnormal_heavy"])
def test_fp8_codes_decode_exactly(codes):
    """Every finite e4m3 code in K and V, or only subnormal / smallest-normal
    codes with a large scale (a flush of subnormals to zero would show)."""
    print(f"case fp8 codes {codes}", flush=True)
    spec = DecodeSpec("codes", 1, 8, 1, 128, 16, "fp8", "bf16", 0.02, lengths=("fixed", 512), seed=9)
    inp = make_inputs(spec)
    rng = np.random.default_rng(0)
    if codes == "all_finite":
        pool = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
        ks, vs, norm = 1.0 / 64, 1.0, 448.0
    else:
        pool = np.array([c for c in range(256) if (c & 0x78) in (0x00, 0x08)], np.uint8)
        ks, vs, norm = 64.0, 64.0, 1.0
    inp.k[...] = rng.choice(pool, size=inp.k.shape)
    inp.v[...] = rng.choice(pool, size=inp.v.shape)
    inp.k_scale[...] = ks
    inp.v_scale[...] = vs
    o_ref, lse_ref = oracle.decode_reference(inp)
    for algo in ("mfma", "valu"):
        o, lse = run_library(inp, algo=algo)
        compare(o / norm, lse, o_ref / norm, lse_ref, "fp8")


# ---------------------------------------------------------------- invariances

def test_page_permutation_is_bitwise_invariant():
    print("case page permutation", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=4, lengths=("list", [70, 900, 2000, 33]))
    a = run_library(make_inputs(spec, perm_seed=1))
    b = run_library(make_inputs(spec, perm_seed=2))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_poisoned_padding_is_bitwise_invisible():
    print("case poison", flush=True)
    for name in ("c4_paged_bf16_b64", "c5_paged_fp8_b128"):
        spec = small_variant(name, batch=3, lengths=("list", [5, 77, 1000]))
        a = run_library(make_inputs(spec, poison=False))
        b = run_library(make_inputs(spec, poison=True))
        np.testing.assert_array_equal(a[0], b[0])
        np.testing.assert_array_equal(a[1], b[1])


def test_repeat_runs_are_bitwise_equal():
    print("case determinism", flush=True)
    spec = small_variant("c5_paged_fp8_b128", batch=3, lengths=("list", [5000, 77, 1000]))
    inp = make_inputs(spec)
    t = to_torch(inp)
    a = run_library(inp, tensors=t)
    b = run_library(inp, tensors=t)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_gqa_matches_mha_with_repeated_heads():
    print("case gqa vs mha", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=2, lengths=("list", [300, 1200]))
    gqa = make_inputs(spec)
    g = spec.group
    mha = dataclasses.replace(gqa, spec=dataclasses.replace(spec, num_kv_heads=spec.num_qo_heads),
                              k=np.repeat(gqa.k, g, axis=2), v=np.repeat(gqa.v, g, axis=2))
    a = run_library(gqa)
    b = run_library(mha)
    assert np.max(np.abs(a[0] - b[0])) <= O_TOL["bf16"]
    o_ref, lse_ref = oracle.decode_reference(gqa)
    compare(*b, o_ref, lse_ref, "bf16")


def test_contiguous_equals_identity_paging():
    print("case contiguous vs paged", flush=True)
    spec_p = DecodeSpec("p", 1, 8, 2, 128, 16, "bf16", "bf16", 0.1, lengths=("fixed", 1234), seed=4)
    spec_c = dataclasses.replace(spec_p, page_size=0)
    a = run_library(make_inputs(spec_p, permute_pages=False))
    b = run_library(make_inputs(spec_c))
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_lse_output_optional_and_stream():
    print("case lse null", flush=True)
    import torch
    import decode_attention_kv_split_amd as kvs

    spec = small_variant("c4_paged_bf16_b64", batch=2, lengths=("list", [100, 3000]))
    inp = make_inputs(spec)
    t = to_torch(inp)
    a, keep = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t["page_indptr"],
                            page_indices=t["page_indices"], kv_len_host=inp.kv_len, sm_scale=spec.sm_scale)
    a.lse = None
    s = torch.cuda.Stream()
    ws = torch.zeros(max(kvs.kvs_decode_workspace_bytes(a), 256), dtype=torch.uint8, device="cuda")  # counters start at zero
    assert kvs.kvs_decode(a, ws.data_ptr(), ws.numel(), s.cuda_stream) == kvs.KVS_OK
    s.synchronize()
    o_ref, lse_ref = oracle.decode_reference(inp)
    o = keep[1].to(torch.float64).cpu().numpy()
    assert np.max(np.abs(o - o_ref)) <= O_TOL["bf16"]


def test_bandwidth_probes():
    print("case probes", flush=True)
    import torch
    import decode_attention_kv_split_amd as kvs

    n = (64 << 20) + 48
    src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
    dst = torch.zeros_like(src)
    s = torch.cuda.current_stream().cuda_stream
    assert kvs.kvs_probe_copy(dst.data_ptr(), src.data_ptr(), n, s) == 0
    assert kvs.kvs_probe_stream_read(src.data_ptr(), n, 0, s) == 0
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    assert kvs.kvs_probe_copy(dst.data_ptr(), src.data_ptr(), 17, s) != 0  # not a multiple of 16


@pytest.mark.parametrize("kv", ["fp8", "bf16"])
@pytest.mark.parametrize("Hk,g,d", [(3, 4, 128), (3, 8, 64), (6, 8, 128), (2, 16, 64)])
def test_kv_head_packing_shapes(kv, Hk, g, d):
    """The packed matrix-core variant: two KV heads per workgroup when the shape
    allows it, one otherwise (odd KV-head counts, groups of 16); per-head fp8
    scales differ inside a pack."""
    print(f"case packing kv={kv} Hk={Hk} g={g} d={d}", flush=True)
    spec = DecodeSpec("pack", 3, Hk * g, Hk, d, 16, kv, "bf16", 1 / math.sqrt(d),
                      lengths=("list", [33, 700, 1500]), seed=Hk * 100 + g + d)
    inp = make_inputs(spec, poison=True)
    for chunk in (0, 48):
        o, lse = run_library(inp, algo="mfma_packed", kv_chunk=chunk)
        o_ref, lse_ref = oracle.decode_reference(inp)
        compare(o, lse, o_ref, lse_ref, kv)


@pytest.mark.parametrize("kv", ["bf16", "fp8"])
def test_large_batch_device_planned(kv):
    """More than 256 requests: the kernels derive the work lists from kv_len on
    the device instead of taking them from the launch arguments."""
    print(f"case large batch {kv}", flush=True)
    spec = DecodeSpec("big", 300, 8, 2, 128, 16, kv, "bf16", 0.1, lengths=("uniform", 0, 700), seed=31)
    inp = make_inputs(spec, poison=True)
    for chunk in (0, 64):
        o, lse = run_library(inp, kv_chunk=chunk)
        o_ref, lse_ref = oracle.decode_reference(inp)
        compare(o, lse, o_ref, lse_ref, kv)


def test_many_items_device_planned():
    """More than 256 splits of one request (16-key chunks of an 8192-key
    request): the work list comes from kv_len on the device."""
    print("case many items", flush=True)
    spec = DecodeSpec("items", 2, 8, 2, 128, 16, "bf16", "bf16", 0.1, lengths=("list", [8192, 300]), seed=32)
    inp = make_inputs(spec, poison=True)
    for algo in ("mfma", "valu"):
        o, lse = run_library(inp, kv_chunk=16, algo=algo)
        o_ref, lse_ref = oracle.decode_reference(inp)
        compare(o, lse, o_ref, lse_ref, "bf16")


def test_python_helpers_single_and_paged():
    """single_decode (one request, contiguous cache, q [Hq, d]) and
    batch_decode_paged (the paged batch) give the oracle's results."""
    import torch
    import decode_attention_kv_split_amd as kvs

    print("case python helpers", flush=True)
    spec = small_variant("c3_llama2_7b_32k", lengths=("fixed", 3000))
    inp = make_inputs(spec)
    t = to_torch(inp)
    o, lse = kvs.single_decode(t["q"][0], t["k"], t["v"], sm_scale=spec.sm_scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_reference(inp)
    compare(o[None].to(torch.float64).cpu().numpy(), lse[None].to(torch.float64).cpu().numpy(), o_ref, lse_ref,
            spec.kv_dtype)

    spec = small_variant("c5_paged_fp8_b128", batch=4, lengths=("list", [5, 600, 2000, 129]))
    inp = make_inputs(spec, poison=True)
    t = to_torch(inp)
    o, lse = kvs.batch_decode_paged(t["q"], t["k"], t["v"], t["page_indptr"], t["page_indices"], t["kv_len"],
                                    kv_len_host=inp.kv_len, sm_scale=spec.sm_scale, k_scale=t["k_scale"],
                                    v_scale=t["v_scale"])
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.decode_reference(inp)
    compare(o.to(torch.float64).cpu().numpy(), lse.to(torch.float64).cpu().numpy(), o_ref, lse_ref, spec.kv_dtype)


@pytest.mark.parametrize("q_len,d", [
    (None, 128),  # decode kernel
    (6, 128),     # 32-column kernel
    (40, 128),    # 32x32 kernel
    (40, 64),     # shared-tile kernel
])
def test_score_spike_after_a_window_start_inside_a_tile(q_len, d):
    """Default settings, a wide score range: the one-row window starts at
    key 29 of a 32-key tile (13 of a 16-key one), and every K row from the
    next tile on is scaled by 8 (exactly, a power of two), so the scores
    after the first few visible keys lie far above theirs and the softmax
    reference moves in mid-stream.  (With two tiles per softmax update in
    the decode kernel this does not leave any lane of a column without keys
    when the reference moves; the unified-max tests force that case.)"""
    print(f"case spike after window start q={q_len} d={d}", flush=True)
    kw = {} if q_len is None else {"q_len": ("fixed", q_len)}
    spec = dataclasses.replace(small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [714, 1530, 362]),
                                             window=301, **kw), head_dim=d, sm_scale=d ** -0.5)
    inp = make_inputs(spec, poison=True)
    k = np.array(inp.k, copy=True)
    P = spec.page_size
    for b in range(spec.batch):
        L = int(inp.kv_len[b])
        n = 1 if inp.qo_indptr is None else int(inp.qo_indptr[b + 1] - inp.qo_indptr[b])
        lo = (max(0, L - n - spec.window + 1) // 32 + 1) * 32  # the next 32-key (and 16-key) tile
        for t in range(lo, L):
            page = int(inp.page_indices[inp.page_indptr[b] + t // P])
            row = (k[page, t % P].astype(np.uint32) << 16).view(np.float32) * np.float32(8.0)
            k[page, t % P] = (row.view(np.uint32) >> 16).astype(np.uint16)
    inp = dataclasses.replace(inp, k=k)
    if inp.qo_indptr is None:
        o_ref, lse_ref = oracle.decode_reference(inp)
    else:
        o_ref, lse_ref = oracle.attention_reference(inp)
    o, lse = run_library(inp, kv_chunk=256)
    compare(o, lse, o_ref, lse_ref, "bf16")
