"""kvs_append (QK-norm, rotary embedding, KV append) against the fp64 oracle
on the GPU, element by element: q_out and the new K/V codes must be the
nearest-even codes of the oracle's values (ties within 2^-16 relative may go
either way), the rest of both pools must be unchanged bit for bit, and
decode attention over the appended cache must match the oracle's attention
over the oracle-appended cache at the decode tolerances."""
import dataclasses

import numpy as np
import pytest

import oracle
from kvs_testlib import _codes_to_torch, check_append, check_codes, compare, run_append, run_library
from workloads import CONFIGS, DecodeSpec, make_append_inputs, small_variant

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import torch
    import decode_attention_kv_split_amd as kvs

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    kvs.load_library()


def _append_then_decode(ai, **kw):
    """Run the append, check it, then attend over the appended cache with
    the appended rows as queries (one per request: decode; several: the
    causal rows of each request) and compare with the oracle's attention
    over the oracle-appended cache."""
    import torch

    got, t = run_append(ai, **kw)
    ref = check_append(ai, got)
    c = ai.cache
    s = c.spec
    codes = oracle.append_codes(ref, s.q_dtype, s.kv_dtype)
    k_pool, v_pool, kv_len = oracle.apply_append(ai, codes)
    after = dataclasses.replace(c, q=codes["q_out"], k=k_pool, v=v_pool, kv_len=kv_len, qo_indptr=ai.qo_indptr)
    o_ref, lse_ref = oracle.attention_reference(after)
    # the GPU attention reads the GPU-appended cache and the GPU's q_out
    t["kv_len"] = torch.from_numpy(kv_len.astype(np.int32)).cuda()
    t["q"] = _codes_to_torch(got["q_out"], s.q_dtype)
    if ai.qo_indptr is not None:
        t["qo_indptr"] = torch.from_numpy(np.asarray(ai.qo_indptr, np.int32)).cuda()
    gpu_after = dataclasses.replace(c, kv_len=kv_len, qo_indptr=ai.qo_indptr)
    o, lse = run_library(gpu_after, tensors=t)
    err, rel = compare(o, lse, o_ref, lse_ref, s.kv_dtype)
    print(f"  attention after append: max|o-o_ref|={err:.2e} lse_rel={rel:.2e}", flush=True)


@pytest.mark.parametrize("name,lens,theta", [
    ("c4_paged_bf16_b64", [0, 15, 16, 31, 300, 2049], 1e4),
    ("c5_paged_fp8_b128", [1, 16, 128, 999, 40], 1e4),
    ("c3_llama2_7b_32k", [333], 1e4),
    ("c1_mha_f32", [512], 1e4),
    ("c2_gemma3_1b", [8191], 1e6),          # global layer
    ("c2_gemma3_1b_w512", [4000], 1e4),     # local layer
])
def test_append_then_decode(name, lens, theta):
    print(f"case append {name} lens={lens} theta={theta}", flush=True)
    spec = small_variant(name, batch=len(lens), lengths=("list", lens))
    _append_then_decode(make_append_inputs(spec, seed=41, theta=theta, poison=True))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("kv", ["bf16", "fp8", "f32"])
def test_append_head_dims_and_pairing(d, interleave, kv):
    print(f"case append d={d} interleave={interleave} kv={kv}", flush=True)
    spec = DecodeSpec("append", 3, 8, 2, d, 16, kv, "f32" if kv == "f32" else "bf16", d ** -0.5,
                      lengths=("list", [5, 16, 100]), seed=7 + d)
    ai = make_append_inputs(spec, theta=1e4, interleave=interleave, poison=True)
    got, _ = run_append(ai)
    check_append(ai, got)


@pytest.mark.parametrize("norm,theta", [(False, 1e4), (True, 0.0), (False, 0.0)])
def test_append_without_norm_or_rope(norm, theta):
    print(f"case append norm={norm} theta={theta}", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [7, 64, 500]))
    ai = make_append_inputs(spec, seed=3, norm=norm, theta=theta, poison=True)
    got, _ = run_append(ai)
    check_append(ai, got)
    if not norm and theta == 0.0:  # a plain copy: q_out is q, the new K/V are the inputs' codes
        assert np.array_equal(got["q_out"], ai.q_new)


def test_append_in_place():
    print("case append in place", flush=True)
    spec = small_variant("c5_paged_fp8_b128", batch=2, lengths=("list", [17, 1000]))
    ai = make_append_inputs(spec, seed=5, poison=True)
    got, _ = run_append(ai, in_place=True)
    check_append(ai, got)


def test_append_far_positions_keep_angle_accuracy():
    """Positions near 65k: the angle pos * theta^(-2j/d) is formed in double
    precision, so the rotation still matches the fp64 oracle to the last bit
    of bf16 (a single-precision angle would be off by ~0.004 rad)."""
    print("case append far positions", flush=True)
    spec = DecodeSpec("far", 1, 4, 1, 256, 0, "bf16", "bf16", 1 / 16, lengths=("fixed", 65535), seed=9)
    for theta in (1e4, 1e6):
        ai = make_append_inputs(spec, theta=theta)
        got, _ = run_append(ai)
        check_append(ai, got)


def test_append_skips_slots_outside_the_page_list():
    """A request whose page list does not reach its new position gets q_out
    but no cache write."""
    print("case append uncovered slot", flush=True)
    spec = small_variant("c4_paged_bf16_b64", batch=2, lengths=("list", [16, 40]))
    ai = make_append_inputs(spec, seed=12, poison=True)
    c = ai.cache
    # drop request 0's reserved page: its list then covers tokens 0..15 only
    indptr = c.page_indptr.copy()
    indices = np.delete(c.page_indices, indptr[1] - 1)
    indptr[1:] -= 1
    cut = dataclasses.replace(ai, cache=dataclasses.replace(c, page_indptr=indptr, page_indices=indices))
    got, _ = run_append(cut)
    ref = oracle.append_reference(cut)
    from kvs_testlib import _term_size
    Q = oracle.decode_codes(cut.q_new, "bf16").reshape(2, 32, 128)
    K = oracle.decode_codes(cut.k_new, "bf16").reshape(2, 8, 128)
    check_codes(got["q_out"], ref["q_out"], "bf16", "q_out", mag=_term_size(cut, Q, cut.q_norm_weight, True))
    raw_before_k = np.asarray(c.k)
    row, slot = oracle.cache_slot(1, 40, 16, indptr, indices)
    mask = np.ones(got["k_pool"].shape[:2], dtype=bool)
    mask[row, slot] = False
    assert np.array_equal(got["k_pool"][mask], raw_before_k[mask])   # request 0 wrote nothing
    check_codes(got["k_pool"][row, slot], ref["k"][1], "bf16", "k[1]",
                mag=_term_size(cut, K, cut.k_norm_weight, True)[1])


@pytest.mark.parametrize("name", ["c4_paged_bf16_b64", "c5_paged_fp8_b128"])
def test_append_full_size(name):
    """The full batch: every q_out row and every new K/V slot against the
    oracle, the pools otherwise unchanged."""
    print(f"case append full {name}", flush=True)
    ai = make_append_inputs(CONFIGS[name], theta=1e4)
    got, _ = run_append(ai)
    check_append(ai, got)


# ------------------------------------------------------------------ INT4 caches, ragged token rows

@pytest.mark.parametrize("interleave", [False, True])
@pytest.mark.parametrize("d", [128, 256])
def test_int4_append_then_decode(d, interleave):
    """New tokens stored into an INT4 cache with each request's existing
    scale (nearest even, saturated to [-8, 7]), then decode over it."""
    print(f"case append int4 d={d} interleave={interleave}", flush=True)
    spec = dataclasses.replace(small_variant("c6_paged_int4_b128", batch=4, lengths=("list", [0, 15, 16, 700])),
                               head_dim=d, sm_scale=d ** -0.5)
    _append_then_decode(make_append_inputs(spec, seed=19 + d, theta=1e4, interleave=interleave, poison=True))


def test_int4_append_saturates():
    """Scales far below the new values: every new code saturates at -8 or 7."""
    print("case append int4 saturation", flush=True)
    spec = small_variant("c6_paged_int4_b128", batch=2, lengths=("list", [30, 3]))
    ai = make_append_inputs(spec, seed=2, theta=1e4, norm=False)
    small = dataclasses.replace(ai.cache, k_scale=np.full_like(ai.cache.k_scale, 1e-3),
                                v_scale=np.full_like(ai.cache.v_scale, 1e-3))
    ai = dataclasses.replace(ai, cache=small)
    got, _ = run_append(ai)
    check_append(ai, got)


@pytest.mark.parametrize("name,rows", [
    ("c4_paged_bf16_b64", [3, 0, 17, 1, 40]),
    ("c5_paged_fp8_b128", [5, 12, 0, 33, 2]),
    ("c6_paged_int4_b128", [8, 1, 21, 0, 64]),
    ("c3_llama2_7b_32k", [100]),
])
def test_ragged_append_then_attend(name, rows):
    """A packed ragged batch of new tokens (0 to 100 per request, paged and
    contiguous, bf16 / fp8 / INT4 caches): every row normed, rotated at its
    own position and stored there, then attention with the appended rows as
    the causal queries of each request."""
    print(f"case append ragged {name} rows={rows}", flush=True)
    lens = [40, 0, 333, 16, 1000][:len(rows)] if len(rows) > 1 else [600]
    spec = small_variant(name, batch=len(rows), lengths=("list", lens))
    _append_then_decode(make_append_inputs(spec, seed=23, theta=1e4, rows=rows, poison=True))


def test_ragged_append_many_requests():
    """300 requests: the request of each token row comes from qo_indptr on
    the device (a binary search) instead of the kernel arguments."""
    print("case append ragged 300 requests", flush=True)
    spec = DecodeSpec("ragged300", 300, 8, 2, 128, 16, "bf16", "bf16", 128 ** -0.5, lengths=("uniform", 0, 300),
                      seed=44)
    rows = np.random.default_rng(1).integers(0, 6, 300)
    _append_then_decode(make_append_inputs(spec, theta=1e4, rows=rows, poison=True))


def test_ragged_append_full_size():
    """The batch-64 paged workload with 4 new tokens per request, every
    output against the oracle."""
    print("case append ragged full c4 x 4", flush=True)
    ai = make_append_inputs(CONFIGS["c4_paged_bf16_b64"], theta=1e4, rows=[4] * 64)
    got, _ = run_append(ai)
    check_append(ai, got)
