"""CPU pins of the multi-token (append / prefill) attention oracle: it
reduces to decode for one query, a fresh prefill's first row sees only key
0, outputs do not depend on later keys (causality), the last row equals
decode over the whole cache, and a window keeps exactly W keys.  Planted
off-by-one positions are caught."""
import dataclasses

import numpy as np
import pytest

import oracle
from oracle import multi as M
from oracle.codecs import decode_codes
from workloads import make_inputs, small_variant


def test_one_query_per_request_is_decode():
    spec = small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [0, 33, 700]))
    inp = make_inputs(spec, poison=True)
    o1, l1 = oracle.decode_reference(inp)
    o2, l2 = oracle.attention_reference(inp)
    assert np.array_equal(o1, o2, equal_nan=True) and np.array_equal(l1, l2, equal_nan=True)


def _prefill(n=40, window=-1, name="c3_llama2_7b_32k"):
    spec = dataclasses.replace(small_variant(name, lengths=("fixed", n), q_len=("fixed", n)), window=window)
    return make_inputs(spec)


def test_fresh_prefill_first_row_sees_key_zero_only():
    inp = _prefill()
    o, lse = oracle.attention_reference(inp)
    V = decode_codes(inp.v, "bf16")        # [L, Hk, d] contiguous
    K = decode_codes(inp.k, "bf16")
    Q = decode_codes(inp.q, "bf16").reshape(40, 32, 128)
    for h in range(32):
        assert np.array_equal(o[0, h], V[0, h])
        assert lse[0, h] == pytest.approx(inp.spec.sm_scale * (Q[0, h] @ K[0, h]), abs=1e-12)


def test_outputs_do_not_depend_on_later_keys():
    inp = _prefill()
    o, lse = oracle.attention_reference(inp)
    k2, v2 = inp.k.copy(), inp.v.copy()
    k2[25:] ^= np.uint16(0x1234)           # scramble the keys and values after position 24
    v2[25:] ^= np.uint16(0x0F0F)
    o2, lse2 = oracle.attention_reference(dataclasses.replace(inp, k=k2, v=v2))
    assert np.array_equal(o[:25], o2[:25]) and np.array_equal(lse[:25], lse2[:25])
    assert not np.allclose(o[25:], o2[25:])


def test_last_row_is_decode_over_the_whole_cache():
    spec = small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [5, 300, 1000]), q_len=("list", [5, 7, 1]))
    inp = make_inputs(spec, poison=True)
    o, lse = oracle.attention_reference(inp)
    last = inp.qo_indptr[1:] - 1
    dec = dataclasses.replace(inp, q=inp.q[last], qo_indptr=None)
    od, ld = oracle.decode_reference(dec)
    assert np.allclose(o[last], od, rtol=0, atol=1e-15) and np.allclose(lse[last], ld, rtol=0, atol=1e-15)


def test_window_keeps_w_keys():
    assert M.query_range(100, 10, 0, 16) == (75, 91)
    assert M.query_range(100, 10, 9, 16) == (84, 100)   # position 99: keys 84..99
    assert M.query_range(10, 10, 3, 16) == (0, 4)
    assert M.query_range(10, 10, 3, -1) == (0, 4)
    inp = _prefill(n=50, window=8)
    o, _ = oracle.attention_reference(inp)
    # a window of 8 at row 30: only keys 23..30 matter
    k2 = inp.k.copy()
    k2[:23] ^= np.uint16(0x2222)
    o2, _ = oracle.attention_reference(dataclasses.replace(inp, k=k2))
    assert np.array_equal(o[30:], o2[30:])      # rows 30.. see keys >= 23 only
    assert not np.allclose(o[29], o2[29])       # row 29's window 22..29 holds a scrambled key


def test_query_lengths_capped_by_kv_len():
    spec = small_variant("c5_paged_fp8_b128", batch=3, lengths=("list", [2, 0, 50]), q_len=("fixed", 4))
    inp = make_inputs(spec)
    assert list(np.diff(inp.qo_indptr)) == [2, 0, 4]
    o, lse = oracle.attention_reference(inp)
    assert o.shape == (6, 64, 128) and np.all(np.isfinite(o))


def test_planted_causal_offset_is_caught(monkeypatch):
    good = M.query_position
    monkeypatch.setattr(M, "query_position", lambda L, n, i: good(L, n, i) + 1)
    with pytest.raises((AssertionError, IndexError, ValueError)):
        test_fresh_prefill_first_row_sees_key_zero_only()
    monkeypatch.setattr(M, "query_position", lambda L, n, i: good(L, n, i) - 1)
    with pytest.raises((AssertionError, IndexError, ValueError)):
        test_last_row_is_decode_over_the_whole_cache()
