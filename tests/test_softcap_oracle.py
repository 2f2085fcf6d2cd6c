"""Pins of the oracle's logit soft-capping, s -> c * tanh(s / c) on the
scaled score (Gemma 2's definition; the pages name the variant without a
formula): a cap too large to act, saturated scores with a closed-form
result, an independent logistic form of tanh, the bound every capped score
obeys, and the chunked form against the direct one."""
import dataclasses
import math

import numpy as np
import pytest
from scipy.special import expit, logsumexp, softmax

import oracle
import oracle.decode as od
from workloads import DecodeSpec, make_inputs, small_variant


def _spec(cap, **kw):
    base = dict(name="cap", batch=1, num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=0, kv_dtype="f32",
                q_dtype="f32", sm_scale=0.125, lengths=("fixed", 77), seed=17, soft_cap=cap)
    base.update(kw)
    return DecodeSpec(**base)


def test_a_huge_cap_does_nothing():
    inp = make_inputs(_spec(0.0))   # cap 0: no cap
    o0, l0 = oracle.decode_reference(inp)
    big = dataclasses.replace(inp, spec=dataclasses.replace(inp.spec, soft_cap=1e9))
    o2, l2 = oracle.decode_reference(big)
    assert np.max(np.abs(o2 - o0)) < 1e-12 and np.max(np.abs(l2 - l0)) < 1e-12
    # a cap the scores (|s| < 5 here) stay far below changes them by < s^3 / (3 c^2)
    mid = dataclasses.replace(inp, spec=dataclasses.replace(inp.spec, soft_cap=1e3))
    _, l3 = oracle.decode_reference(mid)
    assert 0 < np.max(np.abs(l3 - l0)) < 125 / 3e6


def _saturated_case(cap, sm_scale, n_pos, n_neg, d=8, seed=3):
    """Keys along one axis with a sign per key and a query so long that
    |s / c| > 100 for every key: tanh is exactly +-1 in float64, so every
    capped score is exactly +c or -c."""
    rng = np.random.default_rng(seed)
    sign = np.array([1.0] * n_pos + [-1.0] * n_neg)
    rng.shuffle(sign)
    n = sign.size
    K = np.zeros((n, d))
    K[:, 0] = sign * (1.0 + rng.random(n))
    K[:, 1:] = rng.standard_normal((n, d - 1)) * 1e-3
    q = np.zeros(d)
    q[0] = 200.0 * cap / sm_scale
    V = rng.standard_normal((n, d))
    return q, K, V, sign


@pytest.mark.parametrize("cap,sm_scale,n_pos,n_neg", [(50.0, 0.125, 5, 9), (30.0, 1.0, 1, 40), (5.0, 0.0625, 16, 16),
                                                       (50.0, 0.125, 0, 7)])
def test_saturated_scores_closed_form(cap, sm_scale, n_pos, n_neg):
    q, K, V, sign = _saturated_case(cap, sm_scale, n_pos, n_neg)
    o, lse = oracle.attend_direct(q, K, V, sm_scale, cap)
    # weights e^{+c} for keys with a positive score, e^{-c} for the others
    w_pos, w_neg = math.exp(cap), math.exp(-cap)
    total = n_pos * w_pos + n_neg * w_neg
    o_ref = (w_pos * V[sign > 0].sum(axis=0) + w_neg * V[sign < 0].sum(axis=0)) / total
    assert abs(lse - math.log(total)) < 1e-12
    assert np.max(np.abs(o - o_ref)) < 1e-12


def _closed_form_holds(cap, sm_scale):
    q, K, V, sign = _saturated_case(cap, sm_scale, 5, 9)
    o, lse = oracle.attend_direct(q, K, V, sm_scale, cap)
    total = 5 * math.exp(cap) + 9 * math.exp(-cap)
    return abs(lse - math.log(total)) < 1e-9


@pytest.mark.parametrize("mistake", [
    lambda s, c: np.tanh(s / c),                 # outer factor c dropped
    lambda s, c: c * np.tanh(s * c) if c else s,  # divide and multiply swapped
    lambda s, c: np.clip(s, -c, c) if c else s,   # hard clip instead of tanh: same saturated limit
])
def test_planted_mistakes_fail_a_pin(monkeypatch, mistake):
    """Each plausible slip in the cap breaks the closed form or the logistic
    form below; the hard clip agrees when saturated, so the logistic pin must
    catch it."""
    monkeypatch.setattr(od, "cap_scores", lambda s, c: mistake(np.asarray(s, np.float64), c))
    caught = not _closed_form_holds(50.0, 0.125) or not _logistic_form_holds(5.0)
    assert caught


def _logistic_form_holds(cap, seed=8):
    """tanh(x) = 2 * sigmoid(2x) - 1, with the library's softmax and
    logsumexp, on moderate scores the cap compresses strongly."""
    rng = np.random.default_rng(seed)
    n, d = 300, 32
    K, V, q = rng.standard_normal((n, d)), rng.standard_normal((n, d)), rng.standard_normal(d) * 2.0
    sm_scale = 0.5
    s = sm_scale * (K @ q)
    capped = cap * (2.0 * expit(2.0 * s / cap) - 1.0)
    o_ref = softmax(capped) @ V
    lse_ref = float(logsumexp(capped))
    o, lse = oracle.attend_direct(q, K, V, sm_scale, cap)
    return np.max(np.abs(o - o_ref)) < 1e-12 and abs(lse - lse_ref) < 1e-12


@pytest.mark.parametrize("cap", [1.0, 5.0, 50.0])
def test_logistic_form(cap):
    assert _logistic_form_holds(cap)


def test_every_capped_score_stays_inside_the_cap():
    """|c tanh(s/c)| < c, so ln n - c < lse < ln n + c whatever q is."""
    rng = np.random.default_rng(4)
    for cap in (1.0, 10.0, 50.0):
        n, d = 200, 16
        K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
        q = rng.standard_normal(d) * 1e3
        _, lse = oracle.attend_direct(q, K, V, 1.0, cap)
        assert math.log(n) - cap < lse < math.log(n) + cap


@pytest.mark.parametrize("sizes", [[77], [16, 61], [5, 5, 5, 62], [1] * 77])
def test_chunked_form_with_cap(sizes):
    inp = make_inputs(_spec(7.5))
    o1, l1 = oracle.decode_reference(inp)
    o2, l2 = oracle.decode_reference(inp, form="chunked", chunker=lambda n: sizes)
    assert np.max(np.abs(o1 - o2)) < 1e-12 and np.max(np.abs(l1 - l2)) < 1e-12


def test_several_rows_with_cap_one_row_each_is_decode():
    spec = dataclasses.replace(small_variant("c4_paged_bf16_b64", batch=3, lengths=("list", [5, 40, 300])),
                               soft_cap=20.0)
    inp = make_inputs(spec)
    o1, l1 = oracle.decode_reference(inp)
    rows = dataclasses.replace(inp, qo_indptr=np.arange(4, dtype=np.int32))
    o2, l2 = oracle.attention_reference(rows)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
