"""Pins of the fp64 oracle against things other than itself.

Each test fixes the oracle to a closed form, a brute-force evaluation with
Python's ``decimal`` / ``math.fsum`` (no numpy), an invariant of the
definition, or hand-derived worked examples (``tests/golden``).  The last
block plants plausible mistakes into the oracle and checks that some pin
catches each one.
"""
import ast
import dataclasses
import decimal
import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.decode as od
from workloads import DecodeSpec, make_inputs, small_variant

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.json")
D = decimal.Decimal


# ----------------------------------------------------------------------------
# helpers: exact decimal evaluation
# ----------------------------------------------------------------------------

def _dec_eval(expr: str, ctx) -> decimal.Decimal:
    """Evaluate a closed-form expression with e, ln, exp and + - * / only."""
    tree = ast.parse(expr, mode="eval")

    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.Constant):
            return D(str(node.value))
        if isinstance(node, ast.Name):
            if node.id == "e":
                return ctx.exp(D(1))
            raise ValueError(node.id)
        if isinstance(node, ast.UnaryOp) and isinstance(node.op, ast.USub):
            return -ev(node.operand)
        if isinstance(node, ast.BinOp):
            a, b = ev(node.left), ev(node.right)
            op = type(node.op)
            if op is ast.Add:
                return a + b
            if op is ast.Sub:
                return a - b
            if op is ast.Mult:
                return a * b
            if op is ast.Div:
                return a / b
        if isinstance(node, ast.Call) and isinstance(node.func, ast.Name):
            (arg,) = node.args
            x = ev(arg)
            if node.func.id == "exp":
                return ctx.exp(x)
            if node.func.id == "ln":
                return ctx.ln(x)
        raise ValueError(ast.dump(node))

    with decimal.localcontext(ctx):
        return ev(tree)


def _decimal_attention(q, K, V, sm_scale):
    """lse and o of one query row, in 50-digit decimal, from exact inputs."""
    ctx = decimal.Context(prec=50)
    with decimal.localcontext(ctx):
        sc = D(repr(float(sm_scale)))
        scores = [sc * sum(D(repr(float(a))) * D(repr(float(b))) for a, b in zip(q, k)) for k in K]
        total = sum(ctx.exp(s) for s in scores)
        lse = ctx.ln(total)
        w = [ctx.exp(s - lse) for s in scores]
        o = [sum(wi * D(repr(float(v[j]))) for wi, v in zip(w, V)) for j in range(len(V[0]))]
    return [float(x) for x in o], float(lse)


def _dyadic(rng, shape, scale=8):
    """Small dyadic rationals: exact in binary64 and in decimal."""
    return rng.integers(-4 * scale, 4 * scale + 1, size=shape).astype(np.float64) / scale


# ----------------------------------------------------------------------------
# worked examples and brute force
# ----------------------------------------------------------------------------

def _golden_cases():
    with open(GOLDEN) as f:
        return json.load(f)["examples"]


@pytest.mark.parametrize("ex", _golden_cases(), ids=lambda e: e["name"])
def test_golden_worked_examples(ex):
    ctx = decimal.Context(prec=50)
    sm = float(_dec_eval(ex["sm_scale"], ctx))
    K = np.array(ex["k"], np.float64)
    V = np.array(ex["v"], np.float64)
    for h, qh in enumerate(ex["q"]):
        lse_ref = float(_dec_eval(ex["lse"][h], ctx))
        o_ref = np.array([float(_dec_eval(x, ctx)) for x in ex["o"][h]])
        for o, lse in (oracle.attend_direct(np.array(qh, float), K, V, sm),
                       oracle.attend_chunked(np.array(qh, float), K, V, sm, [1] * len(K), tile=1),
                       oracle.attend_chunked(np.array(qh, float), K, V, sm, [len(K)], tile=2)):
            assert abs(lse - lse_ref) <= 1e-14 * max(1.0, abs(lse_ref))
            np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14 * max(1.0, np.max(np.abs(o_ref))))


@pytest.mark.parametrize("seed", range(12))
def test_bruteforce_decimal(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 17))
    d = int(rng.choice([1, 2, 3, 5, 8]))
    q = _dyadic(rng, d)
    K = _dyadic(rng, (n, d))
    V = _dyadic(rng, (n, d))
    sm = [1.0, 0.5, 0.25, 0.125][seed % 4]
    o_ref, lse_ref = _decimal_attention(q, K, V, sm)
    for o, lse in (oracle.attend_direct(q, K, V, sm),
                   oracle.attend_chunked(q, K, V, sm, [n], tile=3)):
        assert abs(lse - lse_ref) <= 1e-14 * max(1.0, abs(lse_ref))
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
def test_bruteforce_fsum_lse(seed):
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 17))
    scores = rng.uniform(-20, 20, size=n)
    V = rng.standard_normal((n, 4))
    _, lse = oracle.softmax_from_scores(scores, V)
    ref = math.log(math.fsum(math.exp(s) for s in scores))
    assert abs(lse - ref) <= 1e-14 * max(1.0, abs(ref))


# ----------------------------------------------------------------------------
# closed forms
# ----------------------------------------------------------------------------

def test_identical_keys_give_mean_of_v():
    rng = np.random.default_rng(1)
    n, d = 37, 16
    k = rng.standard_normal(d)
    K = np.tile(k, (n, 1))
    V = rng.standard_normal((n, d))
    q = rng.standard_normal(d)
    sm = 0.3
    s = sm * float(q @ k)
    for o, lse in (oracle.attend_direct(q, K, V, sm), oracle.attend_chunked(q, K, V, sm, [5, 13, 19])):
        np.testing.assert_allclose(o, V.mean(axis=0), rtol=1e-14, atol=1e-14)
        assert abs(lse - (s + math.log(n))) <= 1e-14 * max(1.0, abs(lse))


def test_one_dominant_score_selects_its_row():
    rng = np.random.default_rng(2)
    n, d = 50, 8
    q = rng.standard_normal(d)
    K = rng.standard_normal((n, d)) * 0.1
    j = 17
    K[j] = 60.0 * q / float(q @ q)  # score of j = 60 * sm / ... see below
    V = rng.standard_normal((n, d))
    sm = 1.0
    s = sm * (K @ q)
    gap = s[j] - np.max(np.delete(s, j))
    assert gap >= 40.0
    o, lse = oracle.attend_direct(q, K, V, sm)
    bound = n * math.exp(-gap) * np.max(np.abs(V))
    np.testing.assert_allclose(o, V[j], rtol=0, atol=bound + 1e-15)
    assert abs(lse - s[j]) <= n * math.exp(-gap) + 1e-14 * abs(s[j])


def test_zero_query_gives_mean_and_log_n():
    rng = np.random.default_rng(3)
    n, d = 23, 8
    K = rng.standard_normal((n, d))
    V = rng.standard_normal((n, d))
    o, lse = oracle.attend_direct(np.zeros(d), K, V, 0.7)
    np.testing.assert_allclose(o, V.mean(axis=0), rtol=1e-14, atol=1e-15)
    assert abs(lse - math.log(n)) <= 1e-15


def test_single_visible_key():
    rng = np.random.default_rng(4)
    d = 8
    q, k, v = rng.standard_normal(d), rng.standard_normal(d), rng.standard_normal(d)
    o, lse = oracle.attend_direct(q, k[None], v[None], 0.5)
    np.testing.assert_array_equal(o, v)
    assert lse == 0.5 * float(k @ q)


def test_empty_visible_set():
    d = 4
    for o, lse in (oracle.attend_direct(np.ones(d), np.zeros((0, d)), np.zeros((0, d)), 1.0),
                   oracle.attend_chunked(np.ones(d), np.zeros((0, d)), np.zeros((0, d)), 1.0, [])):
        assert lse == -math.inf
        assert np.all(o == 0.0)
    o, lse = oracle.merge_states([(-math.inf, np.zeros(d)), (-math.inf, np.zeros(d))])
    assert lse == -math.inf and np.all(o == 0)


# ----------------------------------------------------------------------------
# invariants
# ----------------------------------------------------------------------------

def _random_row(seed, n=97, d=16):
    rng = np.random.default_rng(seed)
    return rng.standard_normal(d), rng.standard_normal((n, d)) * 2, rng.standard_normal((n, d)), rng


@pytest.mark.parametrize("chunking", ["one", "two", "three", "seven", "singletons", "random"])
@pytest.mark.parametrize("tile", [1, 4, 16, 128])
def test_split_count_invariance(chunking, tile):
    q, K, V, rng = _random_row(5)
    n = K.shape[0]
    if chunking == "one":
        sizes = [n]
    elif chunking == "singletons":
        sizes = [1] * n
    elif chunking == "random":
        cuts = np.sort(rng.choice(np.arange(1, n), size=9, replace=False))
        sizes = list(np.diff(np.concatenate([[0], cuts, [n]])))
    else:
        parts = {"two": 2, "three": 3, "seven": 7}[chunking]
        sizes = [len(a) for a in np.array_split(np.arange(n), parts)]
    o1, l1 = oracle.attend_direct(q, K, V, 0.4)
    o2, l2 = oracle.attend_chunked(q, K, V, 0.4, sizes, tile=tile)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-12)
    assert abs(l2 - l1) <= 1e-12 * max(1.0, abs(l1))


def test_merge_is_associative_and_commutative():
    rng = np.random.default_rng(6)
    states = [(float(rng.uniform(-30, 30)), rng.standard_normal(8)) for _ in range(5)]
    states.append((-math.inf, np.zeros(8)))
    ref_o, ref_l = oracle.merge_states(states)
    perm = [states[i] for i in rng.permutation(len(states))]
    o, l = oracle.merge_states(perm)
    np.testing.assert_allclose(o, ref_o, atol=1e-13)
    assert abs(l - ref_l) <= 1e-13 * abs(ref_l)
    left = oracle.merge_states(states[:3])
    right = oracle.merge_states(states[3:])
    o, l = oracle.merge_states([(left[1], left[0]), (right[1], right[0])])
    np.testing.assert_allclose(o, ref_o, atol=1e-13)
    assert abs(l - ref_l) <= 1e-13 * abs(ref_l)


def test_shift_of_scores():
    rng = np.random.default_rng(7)
    s = rng.uniform(-10, 10, 31)
    V = rng.standard_normal((31, 8))
    o, l = oracle.softmax_from_scores(s, V)
    for c in (-50.0, 3.25, 700.0):
        o2, l2 = oracle.softmax_from_scores(s + c, V)
        np.testing.assert_allclose(o2, o, atol=1e-13)
        assert abs(l2 - (l + c)) <= 1e-13 * max(1.0, abs(l + c))


def test_linearity_in_v():
    q, K, V1, rng = _random_row(8)
    V2 = rng.standard_normal(V1.shape)
    a = 2.5
    o1, _ = oracle.attend_direct(q, K, V1, 0.3)
    o2, _ = oracle.attend_direct(q, K, V2, 0.3)
    o12, _ = oracle.attend_direct(q, K, a * V1 + V2, 0.3)
    np.testing.assert_allclose(o12, a * o1 + o2, atol=1e-13)


# ----------------------------------------------------------------------------
# layouts: paging, GQA, window, fp8 scales
# ----------------------------------------------------------------------------

def _paged_spec(kv="bf16", B=3, Hq=8, Hk=2, d=32, P=16, lengths=("list", [1, 40, 77]), window=-1):
    return DecodeSpec("t", B, Hq, Hk, d, P, kv, "bf16" if kv != "f32" else "f32", 0.2,
                      window=window, lengths=lengths, seed=77)


def test_page_permutation_invariance():
    spec = _paged_spec()
    a = make_inputs(spec, perm_seed=1)
    b = make_inputs(spec, perm_seed=2)
    assert not np.array_equal(a.page_indices, b.page_indices)
    oa, la = oracle.decode_reference(a)
    ob, lb = oracle.decode_reference(b)
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(la, lb)


def test_paged_equals_contiguous():
    spec_p = DecodeSpec("p", 1, 4, 2, 16, 8, "bf16", "bf16", 0.25, lengths=("fixed", 61), seed=9)
    spec_c = dataclasses.replace(spec_p, page_size=0)
    for permute in (False, True):
        p = make_inputs(spec_p, permute_pages=permute)
        c = make_inputs(spec_c)
        np.testing.assert_array_equal(p.q, c.q)
        op, lp = oracle.decode_reference(p)
        oc, lc = oracle.decode_reference(c)
        np.testing.assert_array_equal(op, oc)
        np.testing.assert_array_equal(lp, lc)


def test_poisoned_padding_is_never_read():
    spec = _paged_spec()
    clean = make_inputs(spec)
    dirty = make_inputs(spec, poison=True)
    oc, lc = oracle.decode_reference(clean)
    od_, ld = oracle.decode_reference(dirty)
    assert np.all(np.isfinite(od_))
    np.testing.assert_array_equal(oc, od_)
    np.testing.assert_array_equal(lc, ld)


def test_gqa_equals_mha_with_repeated_kv_heads():
    spec = _paged_spec(Hq=8, Hk=2)
    g = 4
    gqa = make_inputs(spec)
    mha = dataclasses.replace(gqa, spec=dataclasses.replace(spec, num_kv_heads=8),
                              k=np.repeat(gqa.k, g, axis=2), v=np.repeat(gqa.v, g, axis=2))
    o1, l1 = oracle.decode_reference(gqa)
    o2, l2 = oracle.decode_reference(mha)
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(l1, l2)


def test_gqa_heads_use_distinct_kv_heads():
    """Query heads of different groups must see different keys."""
    spec = _paged_spec(Hq=4, Hk=2)
    inp = make_inputs(spec)
    o, _ = oracle.decode_reference(inp)
    # heads 0,1 share kv head 0; heads 2,3 share kv head 1.  Replacing kv head 1's
    # values by zeros must zero heads 2,3 only.
    k2 = inp.k.copy()
    v2 = inp.v.copy()
    v2[:, :, 1, :] = 0
    z = dataclasses.replace(inp, k=k2, v=v2)
    oz, _ = oracle.decode_reference(z)
    np.testing.assert_array_equal(oz[:, :2], o[:, :2])
    assert np.all(oz[:, 2:] == 0)


@pytest.mark.parametrize("W", [1, 5, 16, 39, 40, 100])
def test_window_equals_slice(W):
    L = 40
    spec = DecodeSpec("w", 1, 4, 2, 16, 0, "bf16", "bf16", 0.3, window=W, lengths=("fixed", L), seed=10)
    inp = make_inputs(spec)
    o, lse = oracle.decode_reference(inp)
    lo = max(0, L - W)
    sl = dataclasses.replace(inp, spec=dataclasses.replace(spec, window=-1),
                             k=inp.k[lo:], v=inp.v[lo:], kv_len=np.array([L - lo], np.int32))
    o2, l2 = oracle.decode_reference(sl)
    np.testing.assert_array_equal(o, o2)
    np.testing.assert_array_equal(lse, l2)
    if W == 1:
        V = oracle.decode_codes(inp.v[L - 1], "bf16")
        np.testing.assert_array_equal(o[0], np.repeat(V, 2, axis=0))
    if W >= L:
        full = dataclasses.replace(inp, spec=dataclasses.replace(spec, window=-1))
        o3, l3 = oracle.decode_reference(full)
        np.testing.assert_array_equal(o, o3)


def test_zero_length_request():
    spec = _paged_spec(lengths=("list", [0, 17, 0]))
    inp = make_inputs(spec)
    o, lse = oracle.decode_reference(inp)
    assert np.all(lse[0] == -np.inf) and np.all(lse[2] == -np.inf)
    assert np.all(o[0] == 0) and np.all(o[2] == 0)
    assert np.all(np.isfinite(lse[1]))


def test_fp8_scales_match_library_dequant():
    """fp8 decode equals attention over K, V dequantised through torch's own
    e4m3 cast times the per-(request, kv head) scale, gathered page by page."""
    import torch

    spec = _paged_spec(kv="fp8", lengths=("list", [3, 33, 64]))
    inp = make_inputs(spec)
    o1, l1 = oracle.decode_reference(inp)
    P, g = spec.page_size, spec.group
    qf = torch.from_numpy(inp.q.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    for b in range(spec.batch):
        L = int(inp.kv_len[b])
        pages = inp.page_indices[inp.page_indptr[b]:inp.page_indptr[b + 1]]
        kc = np.concatenate([inp.k[p] for p in pages])[:L]  # [L, Hk, d] codes
        vc = np.concatenate([inp.v[p] for p in pages])[:L]
        kf = torch.from_numpy(kc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        vf = torch.from_numpy(vc).view(torch.float8_e4m3fn).to(torch.float64).numpy()
        kf = kf * inp.k_scale[b].astype(np.float64)[None, :, None]
        vf = vf * inp.v_scale[b].astype(np.float64)[None, :, None]
        for h in range(spec.num_qo_heads):
            o, lse = oracle.attend_direct(qf[b, h], kf[:, h // g], vf[:, h // g], spec.sm_scale)
            np.testing.assert_array_equal(o1[b, h], o)
            assert l1[b, h] == lse


def test_direct_and_chunked_agree_on_workload():
    spec = small_variant("c5_paged_fp8_b128", batch=3, lengths=("list", [130, 1, 300]))
    inp = make_inputs(spec, poison=True)
    o1, l1 = oracle.decode_reference(inp)
    o2, l2 = oracle.decode_reference_chunked(inp, lambda n: [min(64, n - i) for i in range(0, n, 64)])
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(l2, l1, rtol=1e-12)


# ----------------------------------------------------------------------------
# planted mistakes: each must be caught by one of the pins above
# ----------------------------------------------------------------------------

def _fails(fn, *args):
    try:
        fn(*args)
    except AssertionError:
        return True
    return False


def test_planted_gqa_head_map_is_caught(monkeypatch):
    monkeypatch.setattr(od, "kv_head_of", lambda h, g: h % g)
    assert _fails(test_gqa_heads_use_distinct_kv_heads)


def test_planted_window_off_by_one_is_caught(monkeypatch):
    monkeypatch.setattr(od, "visible_range", lambda L, W: (max(0, L - W + 1), L) if W > 0 else (0, L))
    assert _fails(test_window_equals_slice, 1) or _fails(test_window_equals_slice, 5)


def test_planted_rescale_sign_is_caught(monkeypatch):
    real = od.chunk_state

    def wrong(q, K, V, sm, tile=16, soft_cap=0.0):
        d = V.shape[1]
        m, l, acc = -math.inf, 0.0, np.zeros(d)
        for t0 in range(0, K.shape[0], tile):
            s = sm * (K[t0:t0 + tile] @ q)
            nm = max(m, float(np.max(s)))
            r = math.exp(nm - m) if math.isfinite(m) else 0.0  # sign flipped
            w = np.exp(s - nm)
            l = r * l + float(np.sum(w))
            acc = r * acc + w @ V[t0:t0 + tile]
            m = nm
        return m, l, acc

    monkeypatch.setattr(od, "chunk_state", wrong)
    assert _fails(test_split_count_invariance, "seven", 4)
    monkeypatch.setattr(od, "chunk_state", real)


def test_planted_dropped_scale_is_caught(monkeypatch):
    real = od.attend_direct
    monkeypatch.setattr(od, "attend_direct", lambda q, K, V, sm, soft_cap=0.0: real(q, K, V, 1.0, soft_cap))
    monkeypatch.setattr(oracle, "attend_direct", od.attend_direct)
    assert _fails(test_bruteforce_decimal, 1)


def test_planted_page_slot_mixup_is_caught(monkeypatch):
    real = od.request_kv

    def wrong(b, **kw):
        kw = dict(kw)
        if kw.get("page_size", 0):
            idx = np.asarray(kw["page_indices"]).copy()
            s, e = int(kw["page_indptr"][b]), int(kw["page_indptr"][b + 1])
            idx[s:e] = idx[s:e][::-1]  # pages visited in reverse order
            kw["page_indices"] = idx
        return real(b, **kw)

    monkeypatch.setattr(od, "request_kv", wrong)
    assert _fails(test_paged_equals_contiguous)


def test_planted_transposed_operand_is_caught(monkeypatch):
    real = od.softmax_from_scores

    def wrong(scores, values):
        o, lse = real(scores, values)
        return o[::-1].copy(), lse  # output dims reversed

    monkeypatch.setattr(od, "softmax_from_scores", wrong)
    assert _fails(test_golden_worked_examples, _golden_cases()[0])


# ----------------------------------------------------------------------------
# decode_reference_sampled: the per-(request, head) helper of the full-size
# GPU checks, pinned against the whole-batch oracle on interleaved picks
# ----------------------------------------------------------------------------

def _sampled_agrees(fn, kv):
    """fn(inp, picks) must reproduce decode_reference bit for bit on a pick
    list that revisits requests out of order (a stale per-request cache
    would show) and covers every query head of two KV heads (a wrong head
    map would show), on a paged GQA cache with a window."""
    int4 = kv == "int4"
    spec = DecodeSpec("s", 4, 8, 2, 128 if int4 else 32, 16, kv, "bf16", 0.2, window=50,
                      lengths=("list", [90, 0, 33, 200]), seed=31)
    inp = make_inputs(spec, poison=True)
    o_ref, l_ref = oracle.decode_reference(inp)
    picks = [(3, 0), (0, 7), (3, 5), (2, 1), (0, 0), (3, 7), (1, 3), (2, 6), (0, 4), (3, 2)]
    got = fn(inp, picks)
    assert len(got) == len(picks)
    for (b, h), (o, lse) in zip(picks, got):
        np.testing.assert_array_equal(o, o_ref[b, h])
        assert (lse == l_ref[b, h]) or (math.isinf(lse) and math.isinf(l_ref[b, h]))


@pytest.mark.parametrize("kv", ["bf16", "fp8", "int4"])
def test_sampled_reference_matches_whole_batch(kv):
    _sampled_agrees(oracle.decode_reference_sampled, kv)


def test_planted_stale_request_cache_in_sampled_is_caught():
    def stale(inp, picks):  # keeps the first request's K/V for every later pick
        s = inp.spec
        g = s.num_qo_heads // s.num_kv_heads
        Q = oracle.decode_codes(inp.q, s.q_dtype).reshape(s.batch, s.num_qo_heads, s.head_dim)
        f = od._fields(inp)
        kv_cache = None
        out = []
        for b, h in picks:
            if kv_cache is None:
                lo, hi = od.visible_range(int(inp.kv_len[b]), s.window)
                kv_cache = od.request_kv(b, tokens=(lo, hi), **f)
            K, V = kv_cache
            out.append(od.attend_direct(Q[b, h], K[:, h // g], V[:, h // g], s.sm_scale, s.soft_cap))
        return out

    assert _fails(_sampled_agrees, stale, "bf16")


def test_planted_head_map_in_sampled_is_caught():
    def wrong_head(inp, picks):  # KV head h % Hk instead of h // g
        s = inp.spec
        Q = oracle.decode_codes(inp.q, s.q_dtype).reshape(s.batch, s.num_qo_heads, s.head_dim)
        f = od._fields(inp)
        out = []
        for b, h in picks:
            lo, hi = od.visible_range(int(inp.kv_len[b]), s.window)
            K, V = od.request_kv(b, tokens=(lo, hi), **f)
            kh = h % s.num_kv_heads
            out.append(od.attend_direct(Q[b, h], K[:, kh], V[:, kh], s.sm_scale, s.soft_cap))
        return out

    assert _fails(_sampled_agrees, wrong_head, "bf16")
