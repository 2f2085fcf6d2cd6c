"""CPU pins of the pre-attention oracle (encoders, QK-norm, rotary embedding,
KV append).  Each pin is chosen so that a plausible mistake fails it: the
planted-mistake tests at the end patch a wrong variant into the oracle and
check that a pin catches it."""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import append as A
from oracle import codecs as C
from workloads import make_append_inputs, small_variant


# ------------------------------------------------------------------ encoders

def test_bf16_encoder_round_trips_every_code():
    codes = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = C.bf16_to_f64(codes)
    fin = np.isfinite(vals)
    back = C.f64_to_bf16_codes(vals[fin])
    # -0.0 keeps its sign through binary32
    assert np.array_equal(back, codes[fin])


def test_bf16_encoder_ties_go_to_even():
    codes = np.arange(0x0001, 0x7F7F, 7, dtype=np.uint16)  # positive finite, skip the top
    lo = C.bf16_to_f64(codes)
    hi = C.bf16_to_f64(codes + 1)
    mid = (lo + hi) / 2  # exact in binary64
    got = C.f64_to_bf16_codes(mid)
    want = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, want)
    # just off the midpoint goes to the nearer neighbour
    assert np.array_equal(C.f64_to_bf16_codes(np.nextafter(mid, 0)), codes)
    assert np.array_equal(C.f64_to_bf16_codes(np.nextafter(mid, np.inf)), codes + 1)


def test_bf16_encoder_overflow_and_library_agreement():
    mx = (2 - 2.0 ** -7) * 2.0 ** 127
    assert C.f64_to_bf16_codes(np.array([mx]))[0] == 0x7F7F
    assert C.f64_to_bf16_codes(np.array([(2 - 2.0 ** -8) * 2.0 ** 127]))[0] == 0x7F80  # tie, odd -> inf
    x = np.random.default_rng(1).standard_normal(50000).astype(np.float32) * np.float32(37.0)
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(C.f64_to_bf16_codes(x.astype(np.float64)), want)


def test_fp8_encoder_round_trips_every_code():
    codes = np.arange(256, dtype=np.uint8)
    vals = C.fp8_e4m3fn_to_f64(codes)
    fin = np.isfinite(vals)
    assert np.array_equal(C.f64_to_fp8_e4m3fn_codes(vals[fin]), codes[fin])
    assert C.f64_to_fp8_e4m3fn_codes(np.array([np.nan]))[0] == 0x7F


def test_fp8_encoder_ties_saturation_subnormals():
    codes = np.arange(0x01, 0x7E, dtype=np.uint8)  # 0x7E = 448 is the largest finite
    lo = C.fp8_e4m3fn_to_f64(codes)
    hi = C.fp8_e4m3fn_to_f64(codes + 1)
    got = C.f64_to_fp8_e4m3fn_codes((lo + hi) / 2)
    assert np.array_equal(got, np.where(codes % 2 == 0, codes, codes + 1))
    enc = lambda v: int(C.f64_to_fp8_e4m3fn_codes(np.array([v]))[0])
    assert enc(448.0) == 0x7E and enc(464.0) == 0x7E and enc(1e9) == 0x7E and enc(-1e9) == 0xFE
    assert enc(2.0 ** -10) == 0x00          # half the smallest subnormal: tie to even (0)
    assert enc(3 * 2.0 ** -10) == 0x02      # tie between codes 1 and 2
    assert enc(2.0 ** -9) == 0x01 and enc(-2.0 ** -9) == 0x81
    assert enc(-0.0) == 0x80 and enc(0.0) == 0x00


def test_fp8_encoder_agrees_with_torch_cast():
    x = np.random.default_rng(2).standard_normal(20000).astype(np.float32) * np.float32(120.0)
    want = torch.from_numpy(np.clip(x, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(C.f64_to_fp8_e4m3fn_codes(x.astype(np.float64)), want)


# ------------------------------------------------------------------ QK-norm

def test_rms_norm_closed_forms():
    y = A.rms_norm(np.array([3.0, 4.0]), None, 0.0)
    r = math.sqrt((9 + 16) / 2)
    assert np.allclose(y, [3 / r, 4 / r], rtol=0, atol=1e-15)
    x = np.random.default_rng(3).standard_normal((5, 128))
    y = A.rms_norm(x, None, 0.0)
    assert np.allclose(np.mean(y * y, axis=-1), 1.0, rtol=0, atol=1e-13)
    assert np.allclose(A.rms_norm(7.5 * x, None, 0.0), y, rtol=0, atol=1e-13)  # scale invariant
    w = np.random.default_rng(4).standard_normal(128)
    assert np.allclose(A.rms_norm(x, w, 0.0), y * w, rtol=0, atol=1e-13)
    assert np.all(A.rms_norm(np.zeros(64), None, 1e-6) == 0.0)
    # eps enters under the root: mean(x^2) = 1e-6 and eps = 1e-6 halve the square
    z = np.full(16, 1e-3)
    assert np.allclose(A.rms_norm(z, None, 1e-6), z / math.sqrt(2e-6), rtol=1e-14)


# ------------------------------------------------------------------ rotary embedding

@pytest.mark.parametrize("interleave", [False, True])
def test_rope_position_zero_is_identity_and_pairs_keep_norm(interleave):
    x = np.random.default_rng(5).standard_normal((3, 128))
    assert np.array_equal(A.rope(x, 0, 10000.0, interleave), x)
    y = A.rope(x, 1234, 10000.0, interleave)
    a, b = A._pairs(128, interleave)
    assert np.allclose(x[:, a] ** 2 + x[:, b] ** 2, y[:, a] ** 2 + y[:, b] ** 2, rtol=1e-13)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rope_first_and_last_pair_closed_form(d):
    p, theta = 777, 10000.0
    e0 = np.zeros(d)
    e0[0] = 1.0
    y = A.rope(e0, p, theta)
    assert y[0] == pytest.approx(math.cos(p), abs=1e-12) and y[d // 2] == pytest.approx(math.sin(p), abs=1e-12)
    el = np.zeros(d)
    el[d // 2 - 1] = 1.0
    t = p * math.pow(theta, -(d - 2) / d)
    y = A.rope(el, p, theta)
    assert y[d // 2 - 1] == pytest.approx(math.cos(t), abs=1e-12) and y[d - 1] == pytest.approx(math.sin(t), abs=1e-12)
    # interleaved: pair j is (2j, 2j+1)
    y = A.rope(e0, p, theta, interleave=True)
    assert y[0] == pytest.approx(math.cos(p), abs=1e-12) and y[1] == pytest.approx(math.sin(p), abs=1e-12)


def _relative_position_holds(theta=1e6, d=128, interleave=False):
    rng = np.random.default_rng(6)
    q, k = rng.standard_normal(d), rng.standard_normal(d)
    for m, n in [(5, 3), (1000, 20), (40000, 39999), (7, 7)]:
        lhs = A.rope(q, m, theta, interleave) @ A.rope(k, n, theta, interleave)
        rhs = A.rope(q, m - n, theta, interleave) @ k
        if abs(lhs - rhs) > 1e-9 * (1 + abs(rhs)):
            return False
    return True


@pytest.mark.parametrize("theta", [10000.0, 1000000.0])
@pytest.mark.parametrize("interleave", [False, True])
def test_rope_scores_depend_only_on_relative_position(theta, interleave):
    assert _relative_position_holds(theta, 128, interleave)


def test_rope_composes_and_interleave_is_a_permutation():
    x = np.random.default_rng(7).standard_normal(128)
    assert np.allclose(A.rope(A.rope(x, 300, 1e4), 45, 1e4), A.rope(x, 345, 1e4), rtol=0, atol=1e-12)
    # interleaved RoPE = rotate-half RoPE conjugated by the pair permutation
    d = 128
    perm = np.empty(d, dtype=np.int64)  # position in the rotate-half layout of interleaved index
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    xi = np.random.default_rng(8).standard_normal(d)
    xh = np.empty(d)
    xh[perm] = xi
    yh = A.rope(xh, 999, 1e4)
    assert np.allclose(A.rope(xi, 999, 1e4, interleave=True), yh[perm], rtol=0, atol=1e-13)


def test_rope_dual_theta_differ_only_past_the_first_pair():
    x = np.random.default_rng(9).standard_normal(256)
    a, b = A.rope(x, 500, 1e4), A.rope(x, 500, 1e6)
    assert a[0] == b[0] and a[128] == b[128]   # frequency theta^0 = 1 in both
    assert not np.allclose(a[1:128], b[1:128])


# ------------------------------------------------------------------ append

@pytest.mark.parametrize("name", ["c4_paged_bf16_b64", "c5_paged_fp8_b128", "c3_llama2_7b_32k", "c1_mha_f32"])
def test_append_then_attend_equals_attention_over_the_extended_cache(name):
    batch = 1 if name in ("c3_llama2_7b_32k", "c1_mha_f32") else 3
    lens = [37] if batch == 1 else [0, 16, 45]
    spec = small_variant(name, batch=batch, lengths=("list", lens))
    ai = make_append_inputs(spec, seed=31, poison=True, theta=1e6 if name.startswith("c3") else 1e4)
    s = spec
    ref = A.append_reference(ai)
    codes = A.append_codes(ref, s.q_dtype, s.kv_dtype)
    k_pool, v_pool, kv_len = A.apply_append(ai, codes)
    # only the new slots changed (raw bits: the f32 padding is NaN)
    raw = lambda a: a.view(np.uint32) if a.dtype == np.float32 else a
    axes = (1, 2) if s.page_size == 0 else (2, 3)
    diff = np.argwhere(np.any(raw(k_pool) != raw(ai.cache.k), axis=axes) |
                       np.any(raw(v_pool) != raw(ai.cache.v), axis=axes))
    want = {A.cache_slot(b, int(ai.cache.kv_len[b]), s.page_size, ai.cache.page_indptr, ai.cache.page_indices)
            for b in range(s.batch)}
    want = {(r,) if sl is None else (r, sl) for r, sl in want}
    assert {tuple(int(t) for t in x) for x in diff} <= want
    # attention over the appended cache, through the decode oracle
    ci = ai.cache
    after = type(ci)(ci.spec, codes["q_out"], k_pool, v_pool, kv_len, ci.page_indptr, ci.page_indices,
                     ci.k_scale, ci.v_scale)
    o, lse = oracle.decode_reference(after)
    # independently: old logical K/V plus the new row, attended directly
    Q = C.decode_codes(codes["q_out"], s.q_dtype).reshape(s.batch, s.num_qo_heads, s.head_dim)
    f = dict(k=ci.k, v=ci.v, kv_len=ci.kv_len, kv_dtype=s.kv_dtype, page_size=s.page_size,
             page_indptr=ci.page_indptr, page_indices=ci.page_indices, k_scale=ci.k_scale, v_scale=ci.v_scale)
    g = s.num_qo_heads // s.num_kv_heads
    for b in range(s.batch):
        K, V = oracle.request_kv(b, **f)
        kn = C.decode_codes(codes["k"][b], s.kv_dtype)
        vn = C.decode_codes(codes["v"][b], s.kv_dtype)
        if s.kv_dtype == "fp8":
            kn, vn = kn * ci.k_scale[b][:, None], vn * ci.v_scale[b][:, None]
        K = np.concatenate([K, kn[None]])
        V = np.concatenate([V, vn[None]])
        for h in range(s.num_qo_heads):
            o2, l2 = oracle.attend_direct(Q[b, h], K[:, h // g], V[:, h // g], s.sm_scale)
            assert np.allclose(o[b, h], o2, rtol=0, atol=1e-12) and abs(lse[b, h] - l2) < 1e-12


def test_new_token_sees_itself_without_rotation():
    """Query and key of the same position: the rotations cancel in their dot
    product, so it equals the dot product of the normalised vectors."""
    spec = small_variant("c4_paged_bf16_b64", batch=2, lengths=("list", [100, 5000]))
    ai = make_append_inputs(spec, seed=5, theta=1e4)
    ref = A.append_reference(ai)
    Qn = C.decode_codes(ai.q_new, "bf16").reshape(2, 32, 128)
    Kn = C.decode_codes(ai.k_new, "bf16").reshape(2, 8, 128)
    for b in range(2):
        for h in range(32):
            lhs = ref["q_out"][b, h] @ ref["k"][b, h // 4]
            rhs = A.rms_norm(Qn[b, h], ai.q_norm_weight, ai.eps) @ A.rms_norm(Kn[b, h // 4], ai.k_norm_weight, ai.eps)
            assert lhs == pytest.approx(rhs, rel=1e-12, abs=1e-12)


def test_append_position_is_kv_len():
    spec = small_variant("c4_paged_bf16_b64", batch=2, lengths=("list", [15, 16]))
    ai = make_append_inputs(spec, seed=3, norm=False, theta=1e4)
    ref = A.append_reference(ai)
    K = C.decode_codes(ai.k_new, "bf16").reshape(2, 8, 128)
    for b, L in enumerate([15, 16]):
        assert np.allclose(ref["k"][b], A.rope(K[b], L, 1e4), rtol=0, atol=0)
        page, slot = A.cache_slot(b, L, 16, ai.cache.page_indptr, ai.cache.page_indices)
        assert slot == L % 16 and page == ai.cache.page_indices[ai.cache.page_indptr[b] + L // 16]
    # request 1 (16 tokens) needs a second page for its new token
    assert ai.cache.page_indptr[2] - ai.cache.page_indptr[1] == 2


def test_fp8_append_quantises_with_the_existing_scale():
    spec = small_variant("c5_paged_fp8_b128", batch=2, lengths=("list", [300, 40]))
    ai = make_append_inputs(spec, seed=8, theta=1e4)
    ref = A.append_reference(ai)
    codes = A.append_codes(ref, "bf16", "fp8")
    for b in range(2):
        x = ref["k"][b] * ai.cache.k_scale[b][:, None]  # undo the division
        dq = C.fp8_e4m3fn_to_f64(codes["k"][b]) * ai.cache.k_scale[b][:, None]
        step = np.abs(x) * 2.0 ** -3 + 2.0 ** -9 * ai.cache.k_scale[b][:, None]
        sat = np.abs(x) > 448 * ai.cache.k_scale[b][:, None]
        assert np.all((np.abs(dq - x) <= step) | sat)


# ------------------------------------------------------------------ planted mistakes

def test_planted_rope_sign_error_is_caught(monkeypatch):
    good = A.rope

    def bad(x, pos, theta, interleave=False):
        y = good(x, pos, theta, interleave)
        a, b = A._pairs(np.asarray(x).shape[-1], interleave)
        t = A.rope_angles(pos, np.asarray(x).shape[-1], theta)
        x = np.asarray(x, dtype=np.float64)
        y[..., a] = x[..., a] * np.cos(t) + x[..., b] * np.sin(t)  # wrong sign
        return y

    monkeypatch.setattr(A, "rope", bad)
    assert not _relative_position_holds()


def test_planted_frequency_exponent_error_is_caught(monkeypatch):
    monkeypatch.setattr(A, "rope_angles",
                        lambda pos, d, theta: float(pos) * np.power(float(theta), -np.arange(d // 2) / d))
    with pytest.raises(AssertionError):
        test_rope_first_and_last_pair_closed_form(128)


def test_planted_pairing_error_is_caught(monkeypatch):
    monkeypatch.setattr(A, "_pairs", lambda d, interleave: (np.arange(0, d, 2), np.arange(1, d, 2)))
    with pytest.raises(AssertionError):
        test_rope_first_and_last_pair_closed_form(128)


def test_planted_position_error_is_caught(monkeypatch):
    good = A.transform_head
    monkeypatch.setattr(A, "transform_head", lambda x, pos, *r: good(x, pos + 1, *r))
    with pytest.raises(AssertionError):
        test_append_position_is_kv_len()


# ------------------------------------------------------------------ INT4 encoder

def _int4_by_bits(codes):
    """Independent INT4 decode: the byte's bits (numpy's unpackbits, least
    significant first) weighted 1, 2, 4, -8 (two's complement), low nibble
    first."""
    bits = np.unpackbits(np.asarray(codes, np.uint8)[..., None], axis=-1, bitorder="little").astype(np.int64)
    w = np.array([1, 2, 4, -8])
    return np.stack([bits[..., :4] @ w, bits[..., 4:] @ w], -1).reshape(np.shape(codes)[:-1] + (-1,))


def test_int4_encoder_every_code_in_both_nibbles():
    v = np.arange(-8, 8, dtype=np.float64)
    pairs = np.stack(np.meshgrid(v, v, indexing="ij"), -1).reshape(256, 2)  # (element 2i, element 2i + 1)
    codes = C.f64_to_int4_codes(pairs)
    assert codes.shape == (256, 1)
    assert sorted(codes[:, 0].tolist()) == list(range(256))  # every byte once
    np.testing.assert_array_equal(_int4_by_bits(codes), pairs)
    np.testing.assert_array_equal(C.int4_to_f64(codes), pairs)


def test_int4_encoder_ties_and_saturation():
    k = np.arange(-8, 7)
    ties = k + 0.5
    want = np.where(k % 2 == 0, k, k + 1)  # the even neighbour
    got = C.int4_to_f64(C.f64_to_int4_codes(np.repeat(ties, 2)))[0::2]
    np.testing.assert_array_equal(got, want)
    below = C.int4_to_f64(C.f64_to_int4_codes(np.repeat(np.nextafter(ties, -np.inf), 2)))[0::2]
    above = C.int4_to_f64(C.f64_to_int4_codes(np.repeat(np.nextafter(ties, np.inf), 2)))[0::2]
    np.testing.assert_array_equal(below, k)
    np.testing.assert_array_equal(above, k + 1)
    sat = np.array([7.49, 7.5, 8.0, 100.0, -8.49, -8.5, -9.0, -1e9, np.nan, -0.0])
    np.testing.assert_array_equal(C.int4_to_f64(C.f64_to_int4_codes(sat)), [7, 7, 7, 7, -8, -8, -8, -8, 0, 0])


def test_int4_encoder_is_the_nearest_code():
    """Brute force over the 16 values: the nearest, ties to the even one."""
    x = np.random.default_rng(4).uniform(-11, 11, 4000)
    x[:200] = np.round(x[:200] * 2) / 2  # plenty of exact ties
    vals = np.arange(-8, 8, dtype=np.float64)
    dist = np.abs(x[:, None] - vals[None, :])
    best = dist.min(axis=1, keepdims=True)
    cand = np.where(dist == best, vals[None, :], np.nan)
    even = np.where(np.nanmax(np.where(np.abs(cand) % 2 == 0, cand, np.nan), axis=1, initial=-99) > -99,
                    np.nanmax(np.where(np.abs(cand) % 2 == 0, cand, np.nan), axis=1, initial=-99),
                    np.nanmax(cand, axis=1))
    np.testing.assert_array_equal(_int4_by_bits(C.f64_to_int4_codes(x)), even)


# ------------------------------------------------------------------ ragged rows (several new tokens per request)

def _unit_queries(ai, d):
    """Every new q row = e_0 (exactly 1.0 at dimension 0), in q's codes."""
    q = np.zeros(np.shape(ai.q_new)[:-1] + (d,), np.float32)
    q[..., 0] = 1.0
    return torch.from_numpy(q).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_ragged_rows_take_consecutive_positions():
    """q = e_0 with no norm: the first rotation pair turns by the position
    itself (theta^0 = 1), so q_out[0] = cos(p) and q_out[d/2] = sin(p) give
    every row's position in closed form: kv_len[b] + i for row i."""
    import dataclasses

    spec = small_variant("c4_paged_bf16_b64", batch=4, lengths=("list", [15, 0, 40, 7]))
    rows = [3, 2, 0, 5]
    ai = make_append_inputs(spec, seed=12, norm=False, theta=1e4, rows=rows)
    ai = dataclasses.replace(ai, q_new=_unit_queries(ai, 128))
    ref = A.append_reference(ai)
    r = 0
    for b, n in enumerate(rows):
        for i in range(n):
            p = int(ai.cache.kv_len[b]) + i
            assert ref["q_out"][r, 0, 0] == pytest.approx(math.cos(p), abs=1e-12)
            assert ref["q_out"][r, 0, 64] == pytest.approx(math.sin(p), abs=1e-12)
            assert ref["pos"][r] == p and ref["req"][r] == b
            r += 1
    assert r == len(ref["pos"])


def test_one_row_per_request_equals_the_single_token_step():
    spec = small_variant("c5_paged_fp8_b128", batch=3, lengths=("list", [5, 300, 17]))
    one = make_append_inputs(spec, seed=2, theta=1e4)
    rag = make_append_inputs(spec, seed=2, theta=1e4, rows=[1, 1, 1])
    a, b = A.append_reference(one), A.append_reference(rag)
    for key in ("q_out", "k", "v", "pos"):
        np.testing.assert_array_equal(a[key], b[key])


def test_ragged_append_equals_successive_single_token_steps():
    """n rows of one request appended at once = n one-token steps, each at
    the length the previous step left (the one-token reading, pinned above)."""
    import dataclasses

    spec = small_variant("c4_paged_bf16_b64", batch=1, lengths=("list", [14]))
    n = 5
    rag = make_append_inputs(spec, seed=4, theta=1e4, rows=[n])
    ref = A.append_reference(rag)
    codes = A.append_codes(ref, "bf16", "bf16")
    k_all, v_all, kv_all = A.apply_append(rag, codes)
    assert kv_all[0] == 14 + n
    cache = rag.cache
    for i in range(n):
        step = dataclasses.replace(rag, q_new=rag.q_new[i:i + 1], k_new=rag.k_new[i:i + 1],
                                   v_new=rag.v_new[i:i + 1], qo_indptr=None, cache=cache)
        r1 = A.append_reference(step)
        np.testing.assert_array_equal(r1["q_out"][0], ref["q_out"][i])
        c1 = A.append_codes(r1, "bf16", "bf16")
        kp, vp, kl = A.apply_append(step, c1)
        cache = dataclasses.replace(cache, k=kp, v=vp, kv_len=kl)
    np.testing.assert_array_equal(cache.k, k_all)
    np.testing.assert_array_equal(cache.v, v_all)


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int4"])
def test_ragged_append_then_attend(kv):
    """Append a ragged batch, then attend with the same rows as queries:
    equals causal attention over the old logical K/V followed by the new
    rows' decoded codes, computed directly; only the new slots change."""
    name = {"bf16": "c4_paged_bf16_b64", "fp8": "c5_paged_fp8_b128", "int4": "c6_paged_int4_b128"}[kv]
    spec = small_variant(name, batch=3, lengths=("list", [0, 31, 50]))
    rows = [4, 0, 17]
    ai = make_append_inputs(spec, seed=7, theta=1e4, rows=rows, poison=True)
    ref = A.append_reference(ai)
    codes = A.append_codes(ref, "bf16", kv)
    k_pool, v_pool, kv_len = A.apply_append(ai, codes)
    np.testing.assert_array_equal(kv_len, np.asarray(ai.cache.kv_len) + rows)
    ci = ai.cache
    changed = np.argwhere(np.any(k_pool != ci.k, axis=(2, 3)) | np.any(v_pool != ci.v, axis=(2, 3)))
    want = {A.cache_slot(b, p, 16, ci.page_indptr, ci.page_indices) for _, b, p in A.token_rows(ai)}
    assert {(int(a), int(c)) for a, c in changed} <= want
    import dataclasses

    after = dataclasses.replace(ci, q=codes["q_out"], k=k_pool, v=v_pool, kv_len=kv_len, qo_indptr=ai.qo_indptr)
    o, lse = oracle.attention_reference(after)
    s = spec
    g = s.num_qo_heads // s.num_kv_heads
    f = dict(k=ci.k, v=ci.v, kv_len=ci.kv_len, kv_dtype=kv, page_size=16, page_indptr=ci.page_indptr,
             page_indices=ci.page_indices, k_scale=ci.k_scale, v_scale=ci.v_scale)
    Q = C.decode_codes(codes["q_out"], "bf16").reshape(-1, s.num_qo_heads, s.head_dim)
    for r, b, p in A.token_rows(ai):
        K, V = oracle.request_kv(b, **f)  # the old tokens
        first = int(ai.qo_indptr[b])
        kn = C.decode_codes(codes["k"][first:r + 1], kv)
        vn = C.decode_codes(codes["v"][first:r + 1], kv)
        if kv != "bf16":
            kn, vn = kn * ci.k_scale[b][:, None], vn * ci.v_scale[b][:, None]
        K, V = np.concatenate([K, kn]), np.concatenate([V, vn])
        assert K.shape[0] == p + 1
        for h in range(s.num_qo_heads):
            o2, l2 = oracle.attend_direct(Q[r, h], K[:, h // g], V[:, h // g], s.sm_scale)
            assert np.allclose(o[r, h], o2, rtol=0, atol=1e-12) and abs(lse[r, h] - l2) < 1e-12


def test_int4_append_quantises_with_the_existing_scale():
    spec = small_variant("c6_paged_int4_b128", batch=2, lengths=("list", [300, 40]))
    ai = make_append_inputs(spec, seed=8, theta=1e4, rows=[2, 3])
    ref = A.append_reference(ai)
    codes = A.append_codes(ref, "bf16", "int4")
    for r, b, _ in A.token_rows(ai):
        x = ref["k"][r] * ai.cache.k_scale[b][:, None]  # undo the division
        dq = C.int4_to_f64(codes["k"][r]) * ai.cache.k_scale[b][:, None]
        sat = (x > 7.5 * ai.cache.k_scale[b][:, None]) | (x < -8.5 * ai.cache.k_scale[b][:, None])
        assert np.all((np.abs(dq - x) <= 0.5 * ai.cache.k_scale[b][:, None] * (1 + 1e-12)) | sat)


def test_planted_reversed_rows_are_caught(monkeypatch):
    good = A.token_rows

    def reversed_rows(ai):
        out = good(ai)
        by_req = {}
        for r, b, p in out:
            by_req.setdefault(b, []).append(p)
        return [(r, b, by_req[b][len(by_req[b]) - 1 - [x[0] for x in out if x[1] == b].index(r)]) for r, b, p in out]

    monkeypatch.setattr(A, "token_rows", reversed_rows)
    with pytest.raises(AssertionError):
        test_ragged_rows_take_consecutive_positions()


def test_planted_row_position_off_by_one_is_caught(monkeypatch):
    good = A.token_rows
    monkeypatch.setattr(A, "token_rows", lambda ai: [(r, b, p + 1) for r, b, p in good(ai)])
    with pytest.raises(AssertionError):
        test_ragged_rows_take_consecutive_positions()


def test_planted_int4_nibble_order_is_caught(monkeypatch):
    good = C.f64_to_int4_codes

    def swapped(x):
        c = good(x)
        return ((c >> 4) | (c << 4)).astype(np.uint8)

    monkeypatch.setattr(C, "f64_to_int4_codes", swapped)
    with pytest.raises(AssertionError):
        test_int4_encoder_every_code_in_both_nibbles()


def test_planted_int4_half_up_rounding_is_caught(monkeypatch):
    def half_up(x):
        k = np.clip(np.floor(np.asarray(x, np.float64) + 0.5), -8, 7).astype(np.int64) & 0xF
        return (k[..., 0::2] | (k[..., 1::2] << 4)).astype(np.uint8)

    monkeypatch.setattr(C, "f64_to_int4_codes", half_up)
    with pytest.raises(AssertionError):
        test_int4_encoder_ties_and_saturation()


# ------------------------------------------------------------------ the GPU tests' checker, on the CPU

@pytest.mark.parametrize("kv,rows", [("bf16", None), ("fp8", [2, 0, 5]), ("int4", [3, 1, 0]), ("int4", None)])
def test_append_checker_accepts_the_oracle_and_catches_a_slip(kv, rows):
    """check_append (what the GPU append tests run) passes on the oracle's
    own codes laid into the pools, and fails when one stored code is off."""
    from kvs_testlib import check_append

    name = {"bf16": "c4_paged_bf16_b64", "fp8": "c5_paged_fp8_b128", "int4": "c6_paged_int4_b128"}[kv]
    spec = small_variant(name, batch=3, lengths=("list", [5, 40, 16]))
    ai = make_append_inputs(spec, seed=1, theta=1e4, rows=rows, poison=True)
    codes = A.append_codes(A.append_reference(ai), "bf16", kv)
    k_pool, v_pool, _ = A.apply_append(ai, codes)
    got = {"q_out": codes["q_out"], "k_pool": k_pool, "v_pool": v_pool}
    check_append(ai, got)
    r, b, p = A.token_rows(ai)[-1]
    page, slot = A.cache_slot(b, p, 16, ai.cache.page_indptr, ai.cache.page_indices)
    bad = np.array(k_pool, copy=True)
    bad[page, slot, 0, 0] ^= 0x22 if kv == "int4" else 0x02  # a different code
    with pytest.raises(AssertionError):
        check_append(ai, dict(got, k_pool=bad))
