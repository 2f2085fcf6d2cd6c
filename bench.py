#!/usr/bin/env python3
"""Benchmark of one decode-attention step (split-KV partial softmax + merge)
on one MI355X.

Default workload: batched paged GQA decode, batch 64, 32 query / 8 KV heads,
head_dim 128, page size 16, kv_len ~ U[512, 16384], bf16 KV (seeded synthetic
inputs).  One step = one kvs_decode call over the whole batch, inputs already
resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--config NAME]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0  # MI355X HBM3E, published
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 matrix throughput, published
METRIC = "decode-attention \u00b5s/step and achieved HBM GB/s (% of peak), paged GQA batch"
CONFIG_ALIASES = {"c1": "c1_mha_f32", "c2": "c2_gemma3_1b", "c2w": "c2_gemma3_1b_w512",
                  "c3": "c3_llama2_7b_32k", "c4": "c4_paged_bf16_b64", "c5": "c5_paged_fp8_b128",
                  "c6": "c6_paged_int4_b128"}
DEFAULT = "c4_paged_bf16_b64"
# measured beside the default workload: the long-context and the fp8 batched
# paged decodes, which share its >= 70%-of-peak target
EXTRA_CONFIGS = ("c3_llama2_7b_32k", "c5_paged_fp8_b128")
_BYTES = {"f32": 4, "bf16": 2, "fp8": 1, "int4": 0.5}

# HBM bytes per launch of the partial kernel, from two rocprofv3 --pmc passes
# (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch) over the default command of
# each workload, each scaled by the factor the same counter gives for
# kvs_probe_copy of 1 GiB (the counter summaries under profiles/ hold the
# commands and raw figures).  A figure is reported only while the sources
# that decide the partial kernel's memory traffic hash to the digest it was
# measured with (partial_kernel_digest); otherwise traffic is null.
MEASURED_TRAFFIC = {
    ("c4_paged_bf16_b64", "partial_mfma_kernel"):
        {"bytes": 2297291927, "digest": "d53822c022b9899e8f7debb5a0c8b52bc0e22ff7b9ad916aca1c9fefd5213595"},
    ("c5_paged_fp8_b128", "partial_mfma_kernel"):
        {"bytes": 1483218586, "digest": "d53822c022b9899e8f7debb5a0c8b52bc0e22ff7b9ad916aca1c9fefd5213595"},
    ("c3_llama2_7b_32k", "partial_mfma_kernel"):
        {"bytes": 537777903, "digest": "d53822c022b9899e8f7debb5a0c8b52bc0e22ff7b9ad916aca1c9fefd5213595"},
    ("c6_paged_int4_b128", "partial_mfma_kernel"):
        {"bytes": 677645231, "digest": "d53822c022b9899e8f7debb5a0c8b52bc0e22ff7b9ad916aca1c9fefd5213595"},
}


# Sources that decide what the matrix-core decode partial kernel reads and
# writes: the kernel, its shared device code, the planner (chunk sizes,
# workspace), the host code that fills its parameters, and the build flags.
DIGEST_SOURCES = ["build.py", "csrc/decode_mfma.hip", "csrc/mfma_tiles.h", "csrc/kvs_device.h", "csrc/plan.cpp",
                  "csrc/plan.h", "csrc/abi.cpp"]


def code_text(name: str, text: str) -> str:
    """Source text without comments and blank space, so that the digest
    changes with the code and not with its comments."""
    import re

    if name.endswith(".py"):
        text = re.sub(r"(?m)^\s*#.*$", "", text)
    else:
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.strip() for line in text.splitlines() if line.strip())


def partial_kernel_digest() -> str:
    """SHA-256 over the code of DIGEST_SOURCES (comments and blank space
    removed)."""
    import hashlib

    pkg = os.path.join(ROOT, "decode_attention_kv_split_amd")
    h = hashlib.sha256()
    for f in DIGEST_SOURCES:
        h.update(os.path.basename(f).encode())
        with open(os.path.join(pkg, f), encoding="utf-8") as fh:
            h.update(code_text(f, fh.read()).encode())
    return h.hexdigest()


def measured_traffic(config_name: str, kernel: str):
    rec = MEASURED_TRAFFIC.get((config_name, kernel))
    if rec is None or rec["digest"] != partial_kernel_digest():
        return None
    return rec["bytes"]


def query_rows(inp) -> np.ndarray:
    """New query tokens of each request (1 each for decode)."""
    if inp.qo_indptr is None:
        return np.ones(inp.spec.batch, np.int64)
    return np.diff(np.asarray(inp.qo_indptr, np.int64))


def visible_lo(inp) -> np.ndarray:
    """First key any query row of each request sees."""
    s = inp.spec
    L = inp.kv_len.astype(np.int64)
    first_q = L - query_rows(inp)  # position of the first new row
    return np.maximum(0, first_q + 1 - s.window) if s.window > 0 else np.zeros_like(L)


def algorithmic_bytes(inp) -> int:
    """Bytes the method must move once: K and V of every (token, KV head)
    some query row sees (once, however many rows see it), q, o, lse of every
    row, kv_len, the page-table entries it reads and the quantisation
    scales (and qo_indptr with several rows per request)."""
    s = inp.spec
    b_kv, b_q = _BYTES[s.kv_dtype], _BYTES[s.q_dtype]
    L = inp.kv_len.astype(np.int64)
    nq = query_rows(inp)
    lo = np.minimum(visible_lo(inp), L)
    vis = int(np.sum(np.where(nq > 0, L - lo, 0)))
    rows = int(nq.sum())
    kv = int(2 * vis * s.num_kv_heads * s.head_dim * b_kv)
    qo = 2 * rows * s.num_qo_heads * s.head_dim * b_q + 4 * rows * s.num_qo_heads
    meta = 4 * s.batch + (4 * (s.batch + 1) if inp.qo_indptr is not None else 0)
    if s.page_size:
        first = lo // s.page_size
        last = (L + s.page_size - 1) // s.page_size
        meta += 4 * (s.batch + 1) + 4 * int(np.sum(np.where(nq > 0, np.maximum(0, last - first), 0)))
    if s.kv_dtype in ("fp8", "int4"):
        meta += 2 * 4 * s.batch * s.num_kv_heads
    return kv + qo + meta


def attention_flops(inp) -> int:
    """Multiply-adds of the two products, 2 flops each: for every (query
    row, query head) and every key the row sees, head_dim for the score and
    head_dim for the weighted sum of V (4 * head_dim flops per pair)."""
    s = inp.spec
    L = inp.kv_len.astype(np.int64)
    nq = query_rows(inp)
    pairs = 0
    for b in range(s.batch):
        n = int(nq[b])
        if n == 0:
            continue
        pos = L[b] - n + np.arange(n, dtype=np.int64)       # position of each row
        lo = np.maximum(0, pos - s.window + 1) if s.window > 0 else np.zeros(n, np.int64)
        pairs += int(np.sum(pos + 1 - lo))
    return 4 * s.head_dim * s.num_qo_heads * pairs


class HipEvents:
    """hipEvent_t pairs through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    def create(self, n):
        out = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(e)) == 0
            out.append(e.value)
        return out

    def elapsed_ms(self, a, b) -> float:
        assert self.hip.hipEventSynchronize(b) == 0
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return float(ms.value)

    def record(self, e, stream):
        assert self.hip.hipEventRecord(e, ctypes.c_void_p(stream)) == 0

    def destroy(self, evs):
        for e in evs:
            self.hip.hipEventDestroy(e)


def probe_read_gbs(nbytes: int = 4 << 30, reps: int = 10) -> float:
    """Achievable streaming-read bandwidth of this GPU (kvs_probe_stream_read)."""
    import torch
    import decode_attention_kv_split_amd as kvs

    buf = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(2):
        assert kvs.kvs_probe_stream_read(buf.data_ptr(), nbytes, 0, stream) == 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        assert kvs.kvs_probe_stream_read(buf.data_ptr(), nbytes, 0, stream) == 0
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    del buf
    torch.cuda.empty_cache()
    return nbytes / dt / 1e9


def probe_copy(nbytes: int, reps: int) -> dict:
    """kvs_probe_copy over nbytes (read nbytes + write nbytes per launch)."""
    import torch
    import decode_attention_kv_split_amd as kvs

    kvs.load_library()
    nbytes = nbytes // 16 * 16
    src = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream().cuda_stream
    assert kvs.kvs_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream) == 0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        assert kvs.kvs_probe_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream) == 0
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    return {"probe": "copy", "bytes_read": nbytes, "bytes_written": nbytes, "us": round(dt * 1e6, 2),
            "GBs": round(2 * nbytes / dt / 1e9, 1)}


def cpu_baseline(inp, budget_s: float = 12.0):
    """The fp64 oracle as it stands, on a bounded sample of the same workload:
    whole requests in order, wrapping round to the first request, until the
    time budget is spent; the rate is the algorithmic bytes of the requests
    done over the time taken."""
    import oracle

    try:
        from threadpoolctl import threadpool_info

        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    s = inp.spec
    L = inp.kv_len.astype(np.int64)
    nq = query_rows(inp)
    lo = np.minimum(visible_lo(inp), L)
    seen = np.where(nq > 0, L - lo, 0)
    vis_all = max(1, int(np.sum(seen)))
    vis = 0
    n_req = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        b = n_req % s.batch
        if inp.qo_indptr is None:
            oracle.decode_reference(inp, requests=[b])
        else:
            oracle.attention_reference(inp, requests=[b])
        vis += int(seen[b])
        n_req += 1
    dt = time.perf_counter() - t0
    frac_bytes = algorithmic_bytes(inp) * (vis / vis_all)
    return {"value": round(frac_bytes / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "us_per_step": round(dt / (vis / vis_all) * 1e6, 1),
            "cpu_model": _cpu_model(), "blas": _blas_vendor(),
            "sample": f"fp64 numpy oracle, {n_req} requests of the {s.batch}-request batch taken in order "
                      f"and wrapping ({vis} visible tokens, {n_req / s.batch:.2f} passes), {dt:.1f} s, "
                      f"same seeded inputs; us_per_step scales the sample to the whole step by visible tokens"}


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or "unknown"


def _blas_vendor() -> str:
    try:
        from threadpoolctl import threadpool_info

        libs = [f"{i.get('internal_api')} {i.get('version')}" for i in threadpool_info() if i.get("user_api") == "blas"]
        return ", ".join(libs) or "unknown"
    except Exception:
        return "unknown"


def cold_steps(step, stream, ev: "HipEvents", nbytes: int, steps: int) -> dict:
    """Device time of single steps bracketed by events, once with each step
    preceded by a read of 1 GiB (more than the 256 MB MALL and the L2s
    together, so the step's inputs are evicted; reading leaves no dirty lines
    to write back during the step) and once without, so that the difference
    is the cache effect alone."""
    import torch

    flush = torch.ones(1 << 28, dtype=torch.int32, device="cuda")  # 1 GiB

    def timed(cold: bool):
        evs = ev.create(2 * steps)
        for i in range(steps):
            if cold:
                flush.max()
            ev.record(evs[2 * i], stream)
            step()
            ev.record(evs[2 * i + 1], stream)
        torch.cuda.synchronize()
        us = np.array([ev.elapsed_ms(evs[2 * i], evs[2 * i + 1]) * 1e3 for i in range(steps)])
        ev.destroy(evs)
        p10, p50, p90 = np.percentile(us, [10, 50, 90])
        return {"step_us_p10_p50_p90": [round(float(x), 2) for x in (p10, p50, p90)],
                "GBs_at_median": round(nbytes / (p50 * 1e-6) / 1e9, 1)}

    out = {"steps": steps, "flushed": timed(True), "not_flushed": timed(False)}
    del flush
    torch.cuda.empty_cache()
    return out


def graph_steps(a, ws, steps: int) -> float:
    """Microseconds per step over `steps` replays of one kvs_decode call
    captured in a HIP graph (host launch cost out of the loop)."""
    import torch

    import decode_attention_kv_split_amd as kvs

    a.prof_events[0] = a.prof_events[1] = None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # one eager call on the side stream before capture
        st = kvs.kvs_decode(a, ws.data_ptr(), ws.numel(), side.cuda_stream)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        st = kvs.kvs_decode(a, ws.data_ptr(), ws.numel(), torch.cuda.current_stream().cuda_stream)
    if st != kvs.KVS_OK:
        raise kvs.KvsError(st)
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / steps


def run(config_name: str, steps: int, warmup: int, algo: str = "auto", kv_chunk: int = 0,
        with_cpu: bool = True, events: bool = True, cold: bool = False, unified_max=None,
        q_len: int = 1, soft_cap: float = 0.0, kv_len: int = 0, graph: bool = False, probe: bool = True,
        merge_mode: str = "auto", wave_split: str = "auto", pool_offset: int = 0, seed=None) -> dict:
    import dataclasses

    import torch

    import decode_attention_kv_split_amd as kvs
    from workloads import CONFIGS, make_inputs

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from kvs_testlib import to_torch

    kvs.load_library()
    spec = CONFIGS[config_name]
    if q_len != 1:
        spec = dataclasses.replace(spec, q_len=("fixed", q_len))
    if soft_cap:
        spec = dataclasses.replace(spec, soft_cap=soft_cap)
    if kv_len:
        spec = dataclasses.replace(spec, lengths=("fixed", kv_len))
    if seed is not None:
        spec = dataclasses.replace(spec, seed=seed)
    t_gen = time.perf_counter()
    inp = make_inputs(spec)
    t = to_torch(inp)
    if pool_offset:
        # the K and V pools placed pool_offset bytes past the start of their allocations
        for name in ("k", "v"):
            x = t[name]
            nb = x.numel() * x.element_size()
            buf = torch.empty(nb + pool_offset, dtype=torch.uint8, device=x.device)
            y = buf[pool_offset:pool_offset + nb].view(x.dtype).view(x.shape)
            y.copy_(x)
            t[name] = y
            t[name + "_buf"] = buf
    t_gen = time.perf_counter() - t_gen
    s = spec
    a, keep = kvs.make_args(t["q"], t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                            page_indices=t.get("page_indices"), kv_len_host=inp.kv_len,
                            k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), sm_scale=s.sm_scale,
                            window=s.window, kv_chunk=kv_chunk, algo=algo, unified_max=unified_max,
                            kv_dtype="int4" if s.kv_dtype == "int4" else None,
                            qo_indptr=t.get("qo_indptr"), qo_indptr_host=inp.qo_indptr,
                            logits_soft_cap=spec.soft_cap, merge_mode=merge_mode, wave_split=wave_split)
    plan = kvs.kvs_decode_plan(a)
    ws = torch.zeros(max(plan.workspace_bytes, 256), dtype=torch.uint8, device="cuda")  # merge counters start at zero
    stream = torch.cuda.current_stream().cuda_stream
    def step(e0=None, e1=None):
        a.prof_events[0] = e0
        a.prof_events[1] = e1
        st = kvs.kvs_decode(a, ws.data_ptr(), ws.numel(), stream)
        if st != kvs.KVS_OK:
            raise kvs.KvsError(st)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # The partial kernel's duration comes from a second pass after the timed
    # one: the kernel's own dispatch stamps a pair of events with its start and
    # end (kvs_decode_args.prof_events), on the stream it runs on.  Stamping
    # costs host time per call, so the timed steps above carry no events.
    part_ms = [float("nan")]
    n_samples = max(20, min(steps, 100)) if events else 0
    if n_samples:
        ev = HipEvents()
        evs = ev.create(2 * n_samples)
        for j in range(n_samples):
            step(evs[2 * j], evs[2 * j + 1])
        torch.cuda.synchronize()
        part_ms = [ev.elapsed_ms(evs[2 * j], evs[2 * j + 1]) for j in range(n_samples)]
        ev.destroy(evs)
    nbytes = algorithmic_bytes(inp)
    ms_per_step = wall * 1e3 / steps
    value = nbytes / (ms_per_step * 1e-3) / 1e9
    part_avg = float(np.mean(part_ms))
    p10, p50, p90 = (float(x) * 1e3 for x in np.percentile(part_ms, [10, 50, 90]))
    achieved = nbytes / (part_avg * 1e-3) / 1e9
    props = torch.cuda.get_device_properties(0)
    kernel = ("partial_valu_kernel" if plan.algo == kvs.KVS_ALGO_VALU else
              "partial_cols32_kernel" if plan.col_share == 2 and s.head_dim == 128 else
              "partial_mfma_kernel" if plan.col_share < 4 else
              "partial_prefill_kernel" if (s.kv_dtype in ("bf16", "fp8", "int4") and s.head_dim == 128)
              or (s.kv_dtype == "bf16" and s.head_dim == 256) else
              "partial_rows_kernel")
    flops = attention_flops(inp)
    # machine balance: bf16 matrix flops per HBM byte at the two published peaks
    mfma_bound = flops / nbytes > PEAK_BF16_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_step": round(ms_per_step * 1e3, 2),
        "pct_of_peak": round(100.0 * value / PEAK_HBM_GBS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{s.kv_dtype} KV, {s.q_dtype} q, fp32 accumulate",
        "data": "synthetic (seeded; N(0,1) K/V, shapes of the named workload)",
        "config": {
            "workload": config_name,
            "batch": s.batch, "num_qo_heads": s.num_qo_heads, "num_kv_heads": s.num_kv_heads,
            "head_dim": s.head_dim, "page_size": s.page_size, "window": s.window, "kv_dtype": s.kv_dtype,
            "sum_kv_len": int(inp.kv_len.sum()), "seed": s.seed,
            "kv_chunk": plan.kv_chunk, "items_per_kv_head": plan.items_per_kv_head,
            "max_splits": plan.max_splits, "merge_in_partial": plan.merge_in_partial,
            "kv_head_packs_per_workgroup": plan.wave_packs, "parallelism": "single GPU",
            "unified_max": unified_max, "q_len": q_len, "soft_cap": spec.soft_cap,
            "kv_len_override": kv_len or None,
            # where the pools sit (a 2 MiB page holds the start of each)
            "kv_pools": {"k_addr": hex(t["k"].data_ptr()), "v_addr": hex(t["v"].data_ptr()),
                         "k_mod_2MiB": t["k"].data_ptr() % (2 << 20), "v_mod_2MiB": t["v"].data_ptr() % (2 << 20),
                         "offset": pool_offset},
        },
        "roofline": {
            "bound": "hbm",
            "kernel": kernel,
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            # the counters were taken in the default configuration of each workload
            "traffic": (measured_traffic(config_name, kernel)
                        if q_len == 1 and not soft_cap and not kv_len and not kv_chunk and algo == "auto"
                        and merge_mode == "auto" and wave_split == "auto" and unified_max is None and not pool_offset
                        else None),
            "kernel_us": round(part_avg * 1e3, 2),
            "kernel_us_p10_p50_p90": [round(p10, 2), round(p50, 2), round(p90, 2)],
            "kernel_launches_timed": n_samples,
            "kernel_timing": "event pairs stamped by the kernel's own dispatch, in a pass after the timed steps",
            "algorithmic_bytes": nbytes,
            "algorithmic_flops": flops,
            "matrix_tflops": round(flops / (part_avg * 1e-3) / 1e12, 2),
        },
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", None),
                   "cus": props.multi_processor_count, "host": platform.node()},
        "partial_kernel_digest": partial_kernel_digest()[:16],
        "probe_stream_read_GBs": round(probe_read_gbs(), 1) if probe else None,
        "input_gen_s": round(t_gen, 1),
    }
    if mfma_bound:  # long prefills: the contraction, not HBM, bounds the kernel
        tf = flops / (part_avg * 1e-3) / 1e12
        out["roofline"].update(bound="mfma", achieved=round(tf, 2), peak=PEAK_BF16_TFLOPS, unit="TFLOP/s",
                               frac=round(tf / PEAK_BF16_TFLOPS, 4))
    if cold:
        out["cold_cache"] = cold_steps(step, stream, HipEvents(), nbytes, max(20, steps // 2))
    if graph:  # the same step replayed from a captured HIP graph
        out["graph_us_per_step"] = round(graph_steps(a, ws, steps), 2)
    if not events:
        out["roofline"].update(achieved=None, frac=None, kernel_us=None, kernel_us_p10_p50_p90=None)
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(inp)
    return out


def summary(rec: dict) -> dict:
    """The per-workload figures of a run() record, for the 'configs' map."""
    r = rec["roofline"]
    c = rec["config"]
    return {"us_per_step": rec["us_per_step"], "value": rec["value"], "unit": rec["unit"],
            "pct_of_peak": rec["pct_of_peak"], "dtype": rec["dtype"],
            "config": {k: c[k] for k in ("batch", "num_qo_heads", "num_kv_heads", "head_dim", "page_size",
                                         "kv_dtype", "sum_kv_len", "seed", "kv_chunk", "items_per_kv_head",
                                         "max_splits", "merge_in_partial", "kv_head_packs_per_workgroup",
                                         "kv_pools")},
            "roofline": {k: r[k] for k in ("bound", "kernel", "achieved", "peak", "unit", "frac", "traffic",
                                           "kernel_us", "kernel_us_p10_p50_p90", "algorithmic_bytes")}}


def append_bytes(ai) -> int:
    """Bytes the pre-attention step must move once: q, k, v of the new token
    in, q_out and the new K/V slots out, the norm weights, kv_len, each
    request's page-table entry (and its indptr pair), fp8 scales."""
    s = ai.cache.spec
    B, Hq, Hk, d = s.batch, s.num_qo_heads, s.num_kv_heads, s.head_dim
    bq, bkv = _BYTES[s.q_dtype], _BYTES[s.kv_dtype]
    n = 2 * B * Hq * d * bq + 2 * B * Hk * d * bq + 2 * B * Hk * d * bkv + 4 * B
    n += 4 * d * ((ai.q_norm_weight is not None) + (ai.k_norm_weight is not None))
    if s.page_size:
        n += 12 * B
    if s.kv_dtype == "fp8":
        n += 2 * 4 * B * Hk
    return n


def run_append_op(config_name: str, steps: int, warmup: int, with_decode: bool, with_cpu: bool,
                  algo: str = "auto") -> dict:
    """Time kvs_append alone (op 'append') or kvs_append followed by
    kvs_decode over the extended cache (op 'step': the attention part of one
    decode step of one layer).  Each call rewrites the same slot, so the
    calls are identical; device kv_len stays the new token's position for the
    append, and a second array holds kv_len + 1 for the decode."""
    import torch

    import decode_attention_kv_split_amd as kvs
    from workloads import CONFIGS, make_append_inputs

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from kvs_testlib import _codes_to_torch, to_torch

    kvs.load_library()
    spec = CONFIGS[config_name]
    theta = 1e6 if config_name == "c2_gemma3_1b" else 1e4
    t_gen = time.perf_counter()
    ai = make_append_inputs(spec, theta=theta)
    t = to_torch(ai.cache)
    t_gen = time.perf_counter() - t_gen
    q = _codes_to_torch(ai.q_new, spec.q_dtype)
    k = _codes_to_torch(ai.k_new, spec.q_dtype)
    v = _codes_to_torch(ai.v_new, spec.q_dtype)
    wq = torch.from_numpy(ai.q_norm_weight).cuda()
    wk = torch.from_numpy(ai.k_norm_weight).cuda()
    aa, keep_a = kvs.make_append_args(q, k, v, t["k"], t["v"], t["kv_len"], page_indptr=t.get("page_indptr"),
                                      page_indices=t.get("page_indices"), k_scale=t.get("k_scale"),
                                      v_scale=t.get("v_scale"), q_norm_weight=wq, k_norm_weight=wk,
                                      norm_eps=ai.eps, rope_theta=ai.theta, rope_interleave=ai.interleave)
    kv_len1 = t["kv_len"] + 1
    host1 = ai.cache.kv_len + 1
    da, keep_d = kvs.make_args(keep_a[0], t["k"], t["v"], kv_len1, page_indptr=t.get("page_indptr"),
                               page_indices=t.get("page_indices"), kv_len_host=host1,
                               k_scale=t.get("k_scale"), v_scale=t.get("v_scale"), sm_scale=spec.sm_scale,
                               window=spec.window, algo=algo)
    ws = torch.zeros(max(kvs.kvs_decode_workspace_bytes(da), 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    def step(e0=None, e1=None):
        aa.prof_events[0], aa.prof_events[1] = e0, e1
        st = kvs.kvs_append(aa, stream)
        if st != kvs.KVS_OK:
            raise kvs.KvsError(st, "kvs_append")
        if with_decode:
            st = kvs.kvs_decode(da, ws.data_ptr(), ws.numel(), stream)
            if st != kvs.KVS_OK:
                raise kvs.KvsError(st)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    # the append kernel's duration: stamped event pairs in a second pass
    n_samples = max(20, min(steps, 100))
    ev = HipEvents()
    evs = ev.create(2 * n_samples)
    for j in range(n_samples):
        step(evs[2 * j], evs[2 * j + 1])
    torch.cuda.synchronize()
    k_ms = [ev.elapsed_ms(evs[2 * j], evs[2 * j + 1]) for j in range(n_samples)]
    ev.destroy(evs)
    nb_append = append_bytes(ai)
    nb = nb_append
    if with_decode:
        after = type(ai.cache)(spec, ai.cache.q, ai.cache.k, ai.cache.v, host1.astype(np.int32),
                               ai.cache.page_indptr, ai.cache.page_indices, ai.cache.k_scale, ai.cache.v_scale)
        nb += algorithmic_bytes(after)
    ms = wall * 1e3 / steps
    kus = float(np.mean(k_ms)) * 1e3
    out = {
        "metric": ("kvs_append (QK-norm + RoPE + KV append) " if not with_decode else
                   "kvs_append + kvs_decode (attention part of one decode step) ") + "us/call and achieved HBM GB/s",
        "value": round(nb / (ms * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup,
        "ms_per_step": round(ms, 5), "us_per_step": round(ms * 1e3, 2),
        "pct_of_peak": round(100.0 * nb / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": f"{spec.q_dtype} q/k/v in, {spec.kv_dtype} cache, fp32 arithmetic (angles fp64)",
        "data": "synthetic (seeded; N(0,1) new token, QK-norm weights N(1, 0.25), theta %g)" % theta,
        "config": {"workload": config_name, "op": "step" if with_decode else "append", "batch": spec.batch,
                   "num_qo_heads": spec.num_qo_heads, "num_kv_heads": spec.num_kv_heads,
                   "head_dim": spec.head_dim, "page_size": spec.page_size, "kv_dtype": spec.kv_dtype},
        "roofline": {"bound": "hbm", "kernel": "append_kernel", "achieved": round(nb_append / (kus * 1e-6) / 1e9, 2),
                     "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(nb_append / (kus * 1e-6) / 1e9 / PEAK_HBM_GBS, 5),
                     "traffic": None, "kernel_us": round(kus, 2), "algorithmic_bytes": nb_append,
                     "kernel_launches_timed": n_samples,
                     "kernel_timing": "event pairs stamped by the kernel's own dispatch, after the timed steps",
                     "note": "a few MB per call: launch-latency-bound, far below the HBM roofline"},
        "input_gen_s": round(t_gen, 1),
    }
    if with_cpu:
        import oracle

        n, t0 = 0, time.perf_counter()
        while time.perf_counter() - t0 < 5.0:
            oracle.append_reference(ai)
            n += 1
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(nb_append * n / dt / 1e9, 5), "unit": "GB/s", "cores": 1,
                               "kind": "oracle",
                               "sample": f"fp64 oracle append_reference over the whole batch, {n} calls, {dt:.1f} s"}
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT)
    ap.add_argument("--op", default="decode", choices=["decode", "append", "step"],
                    help="decode: the split-KV decode attention (default); append: QK-norm + rotary "
                         "embedding + KV append of the new token; step: append then decode")
    ap.add_argument("--algo", default="auto", choices=["auto", "mfma", "mfma_packed", "valu"])
    ap.add_argument("--kv-chunk", type=int, default=0)
    ap.add_argument("--merge", default="auto", choices=["auto", "in_partial", "kernel"],
                    help="where split partials are merged: chosen by the planner, inside the partial kernel, "
                         "or by a second kernel")
    ap.add_argument("--waves", default="auto", choices=["auto", "heads", "tiles"],
                    help="how a matrix-core decode workgroup's four waves share work: one KV-head pack each "
                         "over the whole chunk, or one pack's tiles")
    ap.add_argument("--pool-offset", type=int, default=0, metavar="BYTES",
                    help="place the K and V pools BYTES past the start of their allocations (multiple of 256)")
    ap.add_argument("--unified-max", type=float, default=None,
                    help="start every chunk's softmax from this reference max (scaled-score units)")
    ap.add_argument("--q-len", type=int, default=1,
                    help="new query tokens per request (1: decode; more: append / speculative-verify attention, "
                         "each row causal over the cache)")
    ap.add_argument("--kv-len", type=int, default=0,
                    help="give every request this cache length (0: the workload's own lengths)")
    ap.add_argument("--soft-cap", type=float, default=0.0,
                    help="logit soft-cap c: scores become c * tanh(s / c) (0: none)")
    ap.add_argument("--seed", type=int, default=None,
                    help="draw the workload from this seed instead of its own (other lengths and values)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    ap.add_argument("--single", action="store_true",
                    help="measure the named workload only (the default run adds records of "
                         + " and ".join(EXTRA_CONFIGS) + " under 'configs')")
    ap.add_argument("--no-events", action="store_true",
                    help="no per-launch kernel timing (the event stamps add host time per call, which "
                         "shows in the step time of launch-bound workloads); roofline timing fields become null")
    ap.add_argument("--cold", action="store_true",
                    help="also time single event-bracketed steps with and without a 1 GiB read before each (caches flushed)")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step replayed from a captured HIP graph (graph_us_per_step)")
    ap.add_argument("--probe-copy", type=int, default=0, metavar="BYTES",
                    help="only run kvs_probe_copy of BYTES bytes (hardware byte-counter calibration)")
    args = ap.parse_args()
    if args.probe_copy:
        print(json.dumps(probe_copy(args.probe_copy, args.steps)), flush=True)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path "
              "(each GPU would run its own requests or KV heads independently).", file=sys.stderr)
        sys.exit(2)
    name = CONFIG_ALIASES.get(args.config, args.config)
    if args.op != "decode":
        res = run_append_op(name, args.steps, args.warmup, args.op == "step", with_cpu=not args.no_cpu,
                            algo=args.algo)
        print(json.dumps(res), flush=True)
        return
    if args.pool_offset % 256 or args.pool_offset < 0:
        sys.exit("--pool-offset must be a non-negative multiple of 256")
    res = run(name, args.steps, args.warmup, args.algo, args.kv_chunk, with_cpu=not args.no_cpu,
              events=not args.no_events, cold=args.cold, unified_max=args.unified_max, q_len=args.q_len,
              soft_cap=args.soft_cap, kv_len=args.kv_len, graph=args.graph, merge_mode=args.merge,
              wave_split=args.waves, pool_offset=args.pool_offset, seed=args.seed)
    plain = (args.seed is None and args.merge == "auto" and args.waves == "auto" and args.algo == "auto" and args.kv_chunk == 0
             and args.unified_max is None and args.q_len == 1 and not args.soft_cap and not args.kv_len
             and not args.cold and not args.graph and not args.pool_offset)
    if name == DEFAULT and plain and not args.single:
        # the other two long-context / batched paged workloads of the 70%-of-peak
        # target, measured the same way in the same process
        import torch

        res["configs"] = {}
        for extra in EXTRA_CONFIGS:
            torch.cuda.empty_cache()
            r = run(extra, args.steps, args.warmup, with_cpu=False, events=not args.no_events, probe=False)
            res["configs"][extra] = summary(r)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
