"""The error bound of the fp16 split-partial formats, on the CPU.

Split partials (o_c, lse_c) of a chunked decode are taken from the fp64
oracle's chunk states, stored in a numpy model of each format, restored and
merged by the oracle's LSE rule; each restored row must stay within 2^-11 of
its largest magnitude (bf16 rounding, 2^-9, would not), and the merged output
within 2^-11 * max|V| of the exact merge:
- row-scaled fp16 (bf16 caches): each row times 2^k with k chosen so that the
  row's largest magnitude lies in [2^14, 2^15), the inverse kept beside it;
- fp16 code averages (fp8 caches): the row before the V scale, which lies
  inside the codes' range (|x| <= 448), the V scale applied after the merge.
Half an fp16 ulp in [2^14, 2^15) is 8, i.e. 2^-11 of a row's largest
magnitude, and a merge is a convex combination of the rows.  A plain fp16
row of V at 2^18 overflows, which is why the bf16 form carries a scale."""
import math

import numpy as np
import pytest

import oracle
from oracle.decode import chunk_state


def _chunk_rows(q, K, V, sm_scale, chunk):
    rows = []
    for t0 in range(0, K.shape[0], chunk):
        m, l, acc = chunk_state(q, K[t0:t0 + chunk], V[t0:t0 + chunk], sm_scale)
        rows.append((m + math.log(l), acc / l) if l > 0 else (-math.inf, np.zeros(V.shape[1])))
    return rows


def _row_scaled(o):
    """Stored fp16 row and its multiplier; restored row."""
    mx = float(np.max(np.abs(o)))
    _, ex = math.frexp(mx)  # mx = f * 2^ex, f in [0.5, 1); 0 gives ex = 0
    k = 15 - min(max(ex, -100), 100)
    stored = (o * 2.0 ** k).astype(np.float16)
    assert np.all(np.isfinite(stored)) and float(np.max(np.abs(stored.astype(np.float64)))) < 2.0 ** 15
    return stored.astype(np.float64) * 2.0 ** -k


def _draw(rng, L, d, exps):
    q = rng.standard_normal(d)
    K = rng.standard_normal((L, d))
    V = rng.standard_normal((L, d)) * np.exp2(exps)[:, None]
    return q, K, V


@pytest.mark.parametrize("scale", ["unit", "big", "tiny", "mixed"])
@pytest.mark.parametrize("chunk", [16, 64, 256])
def test_row_scaled_fp16_partials_bound(scale, chunk):
    rng = np.random.default_rng([7, chunk, len(scale)])
    L, d = 1500, 128
    exps = {"unit": np.zeros(L), "big": np.full(L, 18.0), "tiny": np.full(L, -20.0),
            "mixed": np.where((np.arange(L) // 16) % 2 == 0, 16.0, -16.0)}[scale]
    q, K, V = _draw(rng, L, d, exps)
    rows = _chunk_rows(q, K, V, d ** -0.5, chunk)
    restored = [_row_scaled(o) for _, o in rows]
    for (_, o), r in zip(rows, restored):  # per row: half an ulp at the row's top binade
        assert float(np.max(np.abs(r - o))) <= 2.0 ** -11 * float(np.max(np.abs(o)))
    o_exact, lse_exact = oracle.merge_states(rows)
    o_q, lse_q = oracle.merge_states([(lse, r) for (lse, _), r in zip(rows, restored)])
    assert lse_q == lse_exact
    err = float(np.max(np.abs(o_q - o_exact)))
    assert err <= 2.0 ** -11 * float(np.max(np.abs(V))), err


def test_plain_fp16_rows_of_large_bf16_values_overflow():
    """Without the row scale, V at 2^18 does not fit fp16 (largest 65504)."""
    rng = np.random.default_rng(3)
    q, K, V = _draw(rng, 256, 64, np.full(256, 18.0))
    rows = _chunk_rows(q, K, V, 0.125, 64)
    with np.errstate(over="ignore"):
        assert any(not np.all(np.isfinite(o.astype(np.float16))) for _, o in rows)


@pytest.mark.parametrize("chunk", [16, 64, 256])
def test_fp16_code_averages_bound(chunk):
    """fp8 e4m3 codes (the oracle's exact decode), averaged per chunk in code
    units, stored as plain fp16, merged, then scaled by v_scale."""
    rng = np.random.default_rng([11, chunk])
    L, d = 1500, 128
    codes = rng.integers(0, 256, size=(L, d), dtype=np.uint8)
    codes[(codes & 0x7F) == 0x7F] = 0x3C  # no NaN codes
    Vc = oracle.decode_codes(codes, "fp8")  # exact code values, |x| <= 448
    v_scale = 0.0371
    q, K = rng.standard_normal(d), rng.standard_normal((L, d))
    rows = _chunk_rows(q, K, Vc, d ** -0.5, chunk)
    o_exact, _ = oracle.merge_states(rows)
    o_q, _ = oracle.merge_states([(lse, o.astype(np.float16).astype(np.float64)) for lse, o in rows])
    err = float(np.max(np.abs(o_q - o_exact))) * v_scale
    assert err <= 2.0 ** -11 * float(np.max(np.abs(Vc))) * v_scale, err
