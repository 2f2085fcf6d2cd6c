"""The seeded input generators: reproducibility, length laws, page tables,
poisoning and fp8 scales."""
import dataclasses

import numpy as np
import pytest

from oracle import fp8_e4m3fn_to_f64
from workloads import CONFIGS, DecodeSpec, make_inputs, small_variant


def test_same_seed_same_bits():
    spec = small_variant("c4_paged_bf16_b64", batch=5, lengths=("uniform", 1, 100))
    a, b = make_inputs(spec), make_inputs(spec)
    for f in ("q", "k", "v", "kv_len", "page_indptr", "page_indices"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    c = make_inputs(spec, seed=spec.seed + 1)
    assert not np.array_equal(a.q, c.q)


def test_uniform_lengths_in_range_inclusive():
    spec = dataclasses.replace(CONFIGS["c4_paged_bf16_b64"], batch=20000, head_dim=1, num_qo_heads=1,
                               num_kv_heads=1, lengths=("uniform", 3, 9))
    rng_only = make_inputs(dataclasses.replace(spec, page_size=16), lengths=None)
    L = rng_only.kv_len
    assert L.min() == 3 and L.max() == 9


def test_lognormal_lengths():
    spec = dataclasses.replace(CONFIGS["c5_paged_fp8_b128"], batch=4000, head_dim=16, num_qo_heads=1,
                               num_kv_heads=1, kv_dtype="bf16")
    L = make_inputs(spec).kv_len
    assert L.min() >= 128 and L.max() <= 65536
    # median of the unclipped law is 4096; sampling error of the median ~ 1.25 sigma/sqrt(n)
    assert abs(np.log(np.median(L)) - np.log(4096)) < 5 * 1.25 * 0.8 / np.sqrt(len(L))


def test_page_table_is_a_permutation_of_the_pool():
    spec = small_variant("c4_paged_bf16_b64", batch=7, lengths=("uniform", 1, 200))
    inp = make_inputs(spec)
    P = spec.page_size
    n_pages = (inp.kv_len + P - 1) // P
    np.testing.assert_array_equal(np.diff(inp.page_indptr), n_pages)
    assert sorted(inp.page_indices.tolist()) == list(range(inp.k.shape[0]))


@pytest.mark.parametrize("kv", ["f32", "bf16", "fp8"])
def test_poisoned_padding(kv):
    spec = DecodeSpec("p", 3, 4, 2, 8, 16, kv, "bf16" if kv != "f32" else "f32", 0.3,
                      lengths=("list", [5, 16, 17]), seed=3)
    inp = make_inputs(spec, poison=True)
    for b in range(3):
        L = int(inp.kv_len[b])
        last = inp.page_indices[inp.page_indptr[b + 1] - 1]
        rem = L % 16
        if rem:
            pad = inp.k[last, rem:]
            if kv == "f32":
                assert np.all(np.isnan(pad))
            elif kv == "bf16":
                assert np.all(pad == 0x7FC0)
            else:
                assert np.all(pad == 0x7F)


def test_fp8_scale_is_amax_over_448():
    spec = DecodeSpec("f", 2, 4, 2, 16, 16, "fp8", "bf16", 0.25, lengths=("list", [40, 9]), seed=5)
    inp = make_inputs(spec)
    for b in range(2):
        pages = inp.page_indices[inp.page_indptr[b]:inp.page_indptr[b + 1]]
        codes = np.concatenate([inp.k[p] for p in pages])[:inp.kv_len[b]]
        vals = fp8_e4m3fn_to_f64(codes)
        # the element that set the scale lands exactly on +-448
        assert np.allclose(np.max(np.abs(vals), axis=(0, 2)), 448.0)
        assert np.all(inp.k_scale[b] > 0)
