"""Seeded random decode / append configurations for the parity sweep.

Each case draws one point of the space the library accepts: KV type, head
dimension, group size, number of KV heads, page size (or a contiguous
cache), batch and ragged lengths, window, query rows per request, forced
chunk size, unified max, soft cap, kernel family and score scale.  Only
combinations the C ABI documents as supported are drawn (the CPU test in
tests/test_sweep_plan.py plans every case through the library to prove it).
The draw is fixed by the seed, so a failing case is named by its index and
reruns identically.
"""
from __future__ import annotations

import dataclasses
from typing import List

import numpy as np

from workloads import DecodeSpec

SWEEP_SEED = 20261203
SWEEP_CASES = 150

_VALU_MAX_GROUP = {"f32": 16, "bf16": 16, "fp8": 8}


@dataclasses.dataclass(frozen=True)
class SweepCase:
    index: int
    spec: DecodeSpec
    kv_chunk: int
    algo: str
    unified_max: object  # None or float
    poison_invisible: bool
    merge_mode: str = "auto"
    wave_split: str = "auto"
    num_cus: int = 0  # CU count the call is planned for (0: the device's)

    @property
    def multi(self) -> bool:
        return self.spec.q_len != ("fixed", 1)

    def label(self) -> str:
        s = self.spec
        parts = [f"#{self.index}", s.kv_dtype, f"d{s.head_dim}", f"g{s.group}", f"hk{s.num_kv_heads}",
                 f"P{s.page_size}", f"B{s.batch}"]
        if s.window > 0:
            parts.append(f"W{s.window}")
        if self.multi:
            parts.append("rows")
        if self.kv_chunk:
            parts.append(f"c{self.kv_chunk}")
        if self.unified_max is not None:
            parts.append(f"um{self.unified_max:g}")
        if s.soft_cap:
            parts.append(f"cap{s.soft_cap:g}")
        if self.algo != "auto":
            parts.append(self.algo)
        if self.poison_invisible:
            parts.append("nan")
        if self.merge_mode != "auto":
            parts.append(f"merge-{self.merge_mode}")
        if self.wave_split != "auto":
            parts.append(f"waves-{self.wave_split}")
        if self.num_cus:
            parts.append(f"cus{self.num_cus}")
        return "-".join(parts)


_ORACLE_MACS = 3e8


def _oracle_macs(lens, q_len, window, hq, d) -> float:
    """Multiply-adds of the oracle: every (row, head) against its visible keys."""
    total = 0.0
    for b, L in enumerate(lens):
        n = 1 if q_len == ("fixed", 1) else q_len[1][b]
        pos = int(L) - n + np.arange(n)
        vis = pos + 1 - (np.maximum(0, pos - window + 1) if window > 0 else 0)
        total += float(np.sum(vis)) * hq * 2 * d
    return total


def _pick(rng, seq, p=None):
    return seq[int(rng.choice(len(seq), p=p))]


def draw_case(rng, index: int) -> SweepCase:
    kv = _pick(rng, ["f32", "bf16", "fp8", "int4"], p=[0.1, 0.35, 0.3, 0.25])
    d = _pick(rng, [128, 256]) if kv == "int4" else _pick(rng, [64, 128, 256], p=[0.25, 0.5, 0.25])
    g = _pick(rng, [1, 2, 4, 8, 16])
    hk = _pick(rng, [1, 2, 3, 4, 8])
    if g * hk > 64:
        hk = max(1, 64 // g)
    contiguous = rng.random() < 0.2
    batch = 1 if contiguous else int(rng.integers(1, 6))
    if contiguous:
        P = 0
    elif kv == "int4":
        P = _pick(rng, [16, 32, 64])
    else:
        P = _pick(rng, [1, 2, 4, 8, 16, 16, 16, 32, 64])
    lmax = _pick(rng, [40, 300, 2500, 9000], p=[0.2, 0.35, 0.35, 0.1])
    lens = rng.integers(0, lmax + 1, size=batch)
    for i in range(batch):  # edge lengths now and then
        if rng.random() < 0.15:
            lens[i] = _pick(rng, [0, 1, 15, 16, 17, 63, 64, 65])
    if contiguous and lens[0] == 0:
        lens[0] = 1
    window = -1 if rng.random() < 0.5 else _pick(rng, [1, 2, 7, 16, 31, 100, 513, 2000])
    # matrix-core kernels: bf16 q, pages of 16 or more (or contiguous); INT4 only there
    mfma = kv != "f32" and (P == 0 or P >= 16)
    if not mfma and g > _VALU_MAX_GROUP[kv]:  # the vector kernel's largest group
        g = _VALU_MAX_GROUP[kv]
    multi = mfma and rng.random() < 0.4
    q_len = ("fixed", 1)
    if multi:
        qmax = _pick(rng, [3, 12, 40, 130], p=[0.3, 0.3, 0.3, 0.1])
        q_len = ("list", [int(rng.integers(0, min(int(L), qmax) + 1)) for L in lens])
    # keep the fp64 oracle to about a second: halve the lengths (and the rows
    # they allow) while its multiply-adds exceed the budget
    while _oracle_macs(lens, q_len, window, g * hk, d) > _ORACLE_MACS:
        lens = np.maximum(lens // 2, 1 if contiguous else 0)
        if multi:
            q_len = ("list", [min(n, int(L)) for n, L in zip(q_len[1], lens)])
    chunk = 0 if rng.random() < 0.4 else _pick(rng, [16, 32, 48, 64, 96, 256, 1024, 4096])
    algo = "auto"
    if mfma and not multi and kv != "int4":
        r = rng.random()
        if r < 0.15 and g <= _VALU_MAX_GROUP[kv]:
            algo = "valu"
        elif r < 0.3:
            algo = "mfma_packed"
    matrix = mfma and algo != "valu"
    unified = None
    if matrix and rng.random() < 0.25:
        unified = float(_pick(rng, [-20.0, 0.0, 3.0, 30.0, 200.0]))
    cap = 0.0 if rng.random() < 0.7 else float(_pick(rng, [0.5, 4.0, 30.0]))
    sm = d ** -0.5 * (4.0 if rng.random() < 0.2 else 1.0)
    qk_norm = rng.random() < 0.2
    poison_inv = kv in ("bf16", "fp8") and window > 0 and rng.random() < 0.5
    spec = DecodeSpec(f"sweep{index}", batch, g * hk, hk, d, P, kv, "f32" if kv == "f32" else "bf16", sm,
                      window=window, lengths=("list", [int(x) for x in lens]), qk_rmsnorm=qk_norm,
                      seed=SWEEP_SEED + index, q_len=q_len, soft_cap=cap)
    # where the splits merge and how a workgroup's waves share its work, from
    # streams of their own (the other draws stay as they were); one KV-head
    # pack per wave needs one query row and the packs in fours
    merge = ["auto", "in_partial", "kernel"][int(np.random.default_rng([SWEEP_SEED, index]).integers(0, 3))]
    waves = "auto"
    bytes_per = {"bf16": 2, "fp8": 1, "int4": 0.5}.get(kv, 4)
    packable = (d == 128 if kv == "int4" else d * bytes_per < 256) and 2 * g <= 16 and hk % 2 == 0
    pack = 2 if packable and (algo == "mfma_packed" or (kv == "int4" and algo == "auto")) else 1
    if matrix and not multi and (hk // pack) % 4 == 0 and np.random.default_rng([SWEEP_SEED, index, 1]).random() < 0.6:
        waves = "heads"
    return SweepCase(index, spec, int(chunk), algo, unified, poison_inv, merge, waves)


def sweep_cases(n: int = SWEEP_CASES, seed: int = SWEEP_SEED) -> List[SweepCase]:
    rng = np.random.default_rng(seed)
    return [draw_case(rng, i) for i in range(n)]


ROW_SCALE_SEED = 20261204
ROW_SCALE_CASES = 30


def draw_row_scaled_case(rng, index: int) -> SweepCase:
    """A bf16 decode on the matrix-core decode kernel (one query row, pages of
    16 or more or a contiguous cache) with a forced chunk, planned for one CU:
    every launch of two or more workgroups then stores its split partials as
    row-scaled fp16 rows."""
    d = _pick(rng, [64, 128, 256])
    g = _pick(rng, [1, 2, 4, 8, 16])
    hk = _pick(rng, [1, 2, 4, 8])
    if g * hk > 64:
        hk = max(1, 64 // g)
    contiguous = rng.random() < 0.2
    batch = 1 if contiguous else int(rng.integers(1, 6))
    P = 0 if contiguous else _pick(rng, [16, 32, 64])
    lmax = _pick(rng, [300, 2500, 9000], p=[0.3, 0.5, 0.2])
    lens = rng.integers(1, lmax + 1, size=batch)
    for i in range(batch):
        if rng.random() < 0.15:
            lens[i] = _pick(rng, [1, 15, 16, 17, 63, 64, 65])
    window = -1 if rng.random() < 0.5 else _pick(rng, [1, 7, 16, 31, 100, 513, 2000])
    while _oracle_macs(lens, ("fixed", 1), window, g * hk, d) > _ORACLE_MACS:
        lens = np.maximum(lens // 2, 1)
    chunk = _pick(rng, [16, 32, 48, 64, 96, 256])
    algo = "mfma_packed" if rng.random() < 0.3 else "auto"
    unified = float(_pick(rng, [-20.0, 0.0, 3.0, 30.0])) if rng.random() < 0.2 else None
    cap = 0.0 if rng.random() < 0.7 else float(_pick(rng, [0.5, 4.0, 30.0]))
    sm = d ** -0.5 * (4.0 if rng.random() < 0.2 else 1.0)
    poison_inv = window > 0 and rng.random() < 0.5
    merge = _pick(rng, ["auto", "in_partial", "kernel"])
    packable = d * 2 < 256 and 2 * g <= 16 and hk % 2 == 0
    pack = 2 if packable and algo == "mfma_packed" else 1
    waves = "heads" if (hk // pack) % 4 == 0 and hk >= 4 and rng.random() < 0.5 else "auto"
    spec = DecodeSpec(f"rowscale{index}", batch, g * hk, hk, d, P, "bf16", "bf16", sm, window=window,
                      lengths=("list", [int(x) for x in lens]), qk_rmsnorm=rng.random() < 0.2,
                      seed=ROW_SCALE_SEED + index, soft_cap=cap)
    return SweepCase(index, spec, int(chunk), algo, unified, poison_inv, merge, waves, num_cus=1)


def row_scaled_cases(n: int = ROW_SCALE_CASES, seed: int = ROW_SCALE_SEED) -> List[SweepCase]:
    rng = np.random.default_rng(seed)
    return [draw_row_scaled_case(rng, i) for i in range(n)]
