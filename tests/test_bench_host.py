"""Host-side arithmetic of the benchmark: the algorithmic byte count that
the achieved bandwidth is priced on, checked by hand on small workloads."""
import dataclasses
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
from workloads import DecodeSpec, make_inputs  # noqa: E402


LENS = [10, 40, 100]


def _pages(seen):
    """Page-table entries read: the pages holding keys [L - n, L)."""
    return sum((L + 15) // 16 - (L - n) // 16 for L, n in zip(LENS, seen) if n)


def _spec(**kw):
    base = dict(name="t", batch=3, num_qo_heads=8, num_kv_heads=2, head_dim=64, page_size=16, kv_dtype="bf16",
                q_dtype="bf16", sm_scale=0.125, lengths=("list", [10, 40, 100]), seed=1)
    base.update(kw)
    return DecodeSpec(**base)


def test_decode_bytes_contiguous():
    inp = make_inputs(_spec(batch=1, page_size=0, lengths=("fixed", 100)))
    kv = 2 * 100 * 2 * 64 * 2                      # K and V, 2 KV heads, bf16
    qo = 2 * 8 * 64 * 2 + 4 * 8                    # q and o rows, fp32 lse
    assert bench.algorithmic_bytes(inp) == kv + qo + 4


def test_decode_bytes_paged():
    inp = make_inputs(_spec())
    kv = 2 * sum(LENS) * 2 * 64 * 2
    qo = 2 * 3 * 8 * 64 * 2 + 4 * 3 * 8
    assert bench.algorithmic_bytes(inp) == kv + qo + 4 * 3 + 4 * 4 + 4 * (1 + 3 + 7)


def test_decode_bytes_window():
    inp = make_inputs(_spec(window=32))
    seen = [10, 32, 32]                              # the last 32 keys at most
    kv = 2 * sum(seen) * 2 * 64 * 2
    qo = 2 * 3 * 8 * 64 * 2 + 4 * 3 * 8
    assert _pages(seen) == 1 + 3 + 3
    assert bench.algorithmic_bytes(inp) == kv + qo + 4 * 3 + 4 * 4 + 4 * _pages(seen)


def test_several_rows_read_the_union_of_their_keys_once():
    # rows 3, 0, 5: with window 8, request 0 (L 10, 3 rows) sees keys from
    # position 7 - 8 + 1 = 0; request 1 none; request 2 (L 100, 5 rows) from
    # 95 - 8 + 1 = 88
    inp = make_inputs(_spec(window=8, q_len=("list", [3, 0, 5])))
    seen = [10, 0, 12]
    kv = 2 * sum(seen) * 2 * 64 * 2
    rows = 8
    qo = 2 * rows * 8 * 64 * 2 + 4 * rows * 8
    meta = 4 * 3 + 4 * 4 + 4 * _pages(seen) + 4 * 4   # kv_len, page table, qo_indptr
    assert bench.algorithmic_bytes(inp) == kv + qo + meta
    one = make_inputs(_spec(window=8))
    seen1 = [8, 8, 8]
    assert bench.algorithmic_bytes(one) == (2 * 24 * 2 * 64 * 2 + 2 * 3 * 8 * 64 * 2 + 4 * 3 * 8 + 4 * 3 + 4 * 4
                                            + 4 * _pages(seen1))


def test_quantised_bytes():
    fp8 = make_inputs(dataclasses.replace(_spec(), kv_dtype="fp8"))
    int4 = make_inputs(dataclasses.replace(_spec(head_dim=128), kv_dtype="int4"))
    meta = 4 * 3 + 4 * 4 + 4 * 11 + 2 * 4 * 3 * 2        # kv_len, pages, K and V scales
    assert bench.algorithmic_bytes(fp8) == 2 * 150 * 2 * 64 + 2 * 3 * 8 * 64 * 2 + 4 * 24 + meta
    assert bench.algorithmic_bytes(int4) == 2 * 150 * 2 * 64 + 2 * 3 * 8 * 128 * 2 + 4 * 24 + meta
    assert np.all(bench.query_rows(fp8) == 1)


def test_attention_flops_count_every_visible_pair():
    # decode: each (request, head) sees L keys; 4 * d flops per pair
    inp = make_inputs(_spec())
    assert bench.attention_flops(inp) == 4 * 64 * 8 * sum(LENS)
    # rows 3, 0, 5 with window 8: request 0 (L 10) rows at 7, 8, 9 see 8 keys each;
    # request 2 (L 100) rows at 95..99 see 8 each
    rows = make_inputs(_spec(window=8, q_len=("list", [3, 0, 5])))
    assert bench.attention_flops(rows) == 4 * 64 * 8 * (3 * 8 + 5 * 8)
    # a causal prefill of n = L rows sees 1 + 2 + ... + L pairs
    pre = make_inputs(_spec(batch=1, page_size=0, lengths=("fixed", 100), q_len=("fixed", 100)))
    assert bench.attention_flops(pre) == 4 * 64 * 8 * (100 * 101 // 2)


def test_traffic_digest_follows_code_not_comments():
    src = "int f(int x) { // doubles x\n  return 2 * x; /* a\n  note */\n}\n"
    same = "// header\nint f(int x) {\n\n  return 2 * x;   // twice\n}\n"
    other = "int f(int x) { return 3 * x; }\n"
    assert bench.code_text("k.hip", src) == bench.code_text("k.hip", same)
    assert bench.code_text("k.hip", src) != bench.code_text("k.hip", other)
    assert bench.code_text("b.py", "# flags\nFLAGS = ['-O3']\n") == bench.code_text("b.py", "FLAGS = ['-O3']\n")
    assert len(bench.partial_kernel_digest()) == 64
