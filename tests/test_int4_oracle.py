"""CPU pins of the INT4 KV path of the oracle: the packed-nibble codec
against its definition, the generator's quantisation, and attention over an
INT4 cache against dequantisation written a second, independent way."""
import numpy as np
import pytest

import oracle
from oracle import codecs as C
from workloads import make_inputs, small_variant
import dataclasses


def test_every_byte_decodes_to_two_twos_complement_nibbles():
    b = np.arange(256, dtype=np.uint8)
    v = C.int4_to_f64(b[:, None])          # [256, 2]
    # second derivation: flip the sign bit to offset binary, subtract 8
    lo = ((b & 0xF) ^ 8).astype(np.int64) - 8
    hi = ((b >> 4) ^ 8).astype(np.int64) - 8
    assert np.array_equal(v[:, 0], lo) and np.array_equal(v[:, 1], hi)
    assert tuple(C.int4_to_f64(np.array([0x0F], np.uint8))) == (-1.0, 0.0)
    assert tuple(C.int4_to_f64(np.array([0x87], np.uint8))) == (7.0, -8.0)
    assert tuple(C.int4_to_f64(np.array([0x78], np.uint8))) == (-8.0, 7.0)
    assert v.min() == -8 and v.max() == 7


def test_rows_unpack_in_element_order():
    row = np.array([0x21, 0x43, 0x65, 0x07], np.uint8)   # 1,2,3,4,5,6,7,0
    assert list(C.decode_codes(row, "int4")) == [1, 2, 3, 4, 5, 6, 7, 0]
    assert C.decode_codes(np.zeros((3, 2, 64), np.uint8), "int4").shape == (3, 2, 128)


def test_generator_quantisation_error_and_range():
    spec = small_variant("c6_paged_int4_b128", batch=3, lengths=("list", [40, 300, 17]))
    inp = make_inputs(spec)
    assert inp.k.dtype == np.uint8 and inp.k.shape[-1] == spec.head_dim // 2
    # re-draw the same logical values and compare with the dequantised cache
    f = dict(k=inp.k, v=inp.v, kv_len=inp.kv_len, kv_dtype="int4", page_size=16, page_indptr=inp.page_indptr,
             page_indices=inp.page_indices, k_scale=inp.k_scale, v_scale=inp.v_scale)
    for b in range(3):
        K, V = oracle.request_kv(b, **f)
        codes = K / inp.k_scale[b][None, :, None]
        assert np.allclose(codes, np.rint(codes)) and codes.min() >= -8 and codes.max() <= 7
        # amax maps to +-7
        assert np.allclose(np.max(np.abs(codes), axis=(0, 2)), 7.0)


def test_attention_over_int4_cache_matches_independent_dequantisation():
    spec = small_variant("c6_paged_int4_b128", batch=2, lengths=("list", [33, 200]))
    inp = make_inputs(spec, poison=True)
    o, lse = oracle.decode_reference(inp)
    Q = C.bf16_to_f64(inp.q).reshape(2, 64, 128)
    for b in range(2):
        L = int(inp.kv_len[b])
        pages = inp.page_indices[inp.page_indptr[b]:inp.page_indptr[b + 1]]
        t = np.arange(L)
        kb = inp.k[pages[t // 16], t % 16]              # [L, Hk, 64] bytes
        vb = inp.v[pages[t // 16], t % 16]
        # independent unpack: np.unpackbits, little bit order, two's complement
        def deq(x, s):
            bits = np.unpackbits(x[..., None], axis=-1, bitorder="little")   # [..., 64, 8]
            nib = bits[..., :4] @ (1 << np.arange(4)), bits[..., 4:] @ (1 << np.arange(4))
            out = np.stack([(n ^ 8) - 8 for n in nib], axis=-1).reshape(x.shape[:-1] + (128,))
            return out * s[None, :, None]
        K, V = deq(kb, inp.k_scale[b]), deq(vb, inp.v_scale[b])
        for h in range(64):
            o2, l2 = oracle.attend_direct(Q[b, h], K[:, h // 8], V[:, h // 8], spec.sm_scale)
            assert np.allclose(o[b, h], o2, rtol=0, atol=1e-12) and abs(lse[b, h] - l2) < 1e-12


def test_planted_nibble_order_mistake_is_caught(monkeypatch):
    def swapped(codes):
        c = np.asarray(codes, dtype=np.uint8)
        return C.__dict__["_int4_true"](((c >> 4) | (c << 4)).astype(np.uint8))
    monkeypatch.setitem(C.__dict__, "_int4_true", C.int4_to_f64)
    monkeypatch.setattr(C, "int4_to_f64", swapped)
    with pytest.raises(AssertionError):
        test_rows_unpack_in_element_order()
