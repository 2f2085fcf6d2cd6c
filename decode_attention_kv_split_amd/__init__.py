"""Python binding of libkvsplit (split-KV decode attention on MI355X / gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of ``libkvsplit.so``.  There is no CPU fallback; if the library is
not built, every call raises.

Low level (same names as the C ABI in ``include/kvsplit.h``):
    kvs_decode(args, workspace_ptr, workspace_bytes, stream) -> status
    kvs_decode_noalloc(args, stream) -> status
    kvs_decode_plan(args) -> KvsPlanInfo
    kvs_decode_workspace_bytes(args) -> int
    kvs_append(args, stream) -> status
    kvs_status_string(status) -> str
    kvs_abi_version() -> int
High level, on torch tensors already on the GPU:
    decode(...)              any layout, returns (o, lse)
    single_decode(q, k, v)   one request, contiguous cache
    batch_decode_paged(...)  paged cache
    append(...)              QK-norm, rotary embedding and KV append of the new tokens
"""
from __future__ import annotations

import ctypes
import math
import os
import threading
from typing import Optional, Tuple

__all__ = [
    "KVS_OK", "KVS_ERR_INVALID_ARG", "KVS_ERR_UNSUPPORTED", "KVS_ERR_WORKSPACE", "KVS_ERR_HIP",
    "KVS_ERR_TOO_LARGE", "KVS_NOALLOC_SCRATCH_BYTES", "kvs_decode_noalloc", "KVS_WORKSPACE_COUNTER_BYTES",
    "KVS_F32", "KVS_BF16", "KVS_FP8_E4M3", "KVS_INT4", "KVS_ALGO_AUTO", "KVS_ALGO_VALU", "KVS_ALGO_MFMA",
    "KVS_ALGO_MFMA_PACKED", "KVS_MERGE_AUTO", "KVS_MERGE_IN_PARTIAL", "KVS_MERGE_KERNEL",
    "KVS_WAVES_AUTO", "KVS_WAVES_HEADS", "KVS_WAVES_TILES",
    "KVS_PART_F32", "KVS_PART_F16_CODES", "KVS_PART_F16_ROWS",
    "KvsDecodeArgs", "KvsPlanInfo", "KvsAppendArgs", "KvsError",
    "library_path", "load_library",
    "kvs_decode", "kvs_decode_plan", "kvs_decode_workspace_bytes", "kvs_append", "kvs_status_string",
    "kvs_abi_version", "KVS_ABI_VERSION",
    "kvs_probe_stream_read", "kvs_probe_copy",
    "decode", "single_decode", "batch_decode_paged", "append", "make_append_args",
]

KVS_ABI_VERSION = 12

KVS_OK, KVS_ERR_INVALID_ARG, KVS_ERR_UNSUPPORTED, KVS_ERR_WORKSPACE, KVS_ERR_HIP = 0, -1, -2, -3, -4
KVS_ERR_TOO_LARGE = -5
KVS_NOALLOC_SCRATCH_BYTES = 32 << 20
KVS_WORKSPACE_COUNTER_BYTES = 65536
KVS_F32, KVS_BF16, KVS_FP8_E4M3, KVS_INT4 = 0, 1, 2, 3
KVS_ALGO_AUTO, KVS_ALGO_VALU, KVS_ALGO_MFMA, KVS_ALGO_MFMA_PACKED = 0, 1, 2, 3
KVS_MERGE_AUTO, KVS_MERGE_IN_PARTIAL, KVS_MERGE_KERNEL = 0, 1, 2
_MERGE_MODES = {"auto": KVS_MERGE_AUTO, "in_partial": KVS_MERGE_IN_PARTIAL, "kernel": KVS_MERGE_KERNEL}
KVS_WAVES_AUTO, KVS_WAVES_HEADS, KVS_WAVES_TILES = 0, 1, 2
KVS_PART_F32, KVS_PART_F16_CODES, KVS_PART_F16_ROWS = 0, 1, 2
_WAVE_SPLITS = {"auto": KVS_WAVES_AUTO, "heads": KVS_WAVES_HEADS, "tiles": KVS_WAVES_TILES}
_ALGOS = {"auto": KVS_ALGO_AUTO, "valu": KVS_ALGO_VALU, "mfma": KVS_ALGO_MFMA, "mfma_packed": KVS_ALGO_MFMA_PACKED}

_PKG = os.path.dirname(os.path.abspath(__file__))


def library_path() -> str:
    return os.path.join(_PKG, "_lib", "libkvsplit.so")


class KvsDecodeArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("page_indptr", ctypes.c_void_p),
        ("page_indices", ctypes.c_void_p),
        ("kv_len", ctypes.c_void_p),
        ("kv_len_host", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("sm_scale", ctypes.c_float),
        ("window", ctypes.c_int32),
        ("kv_chunk", ctypes.c_int32),
        ("algo", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("o", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("prof_events", ctypes.c_void_p * 2),
        ("use_unified_max", ctypes.c_int32),
        ("unified_max", ctypes.c_float),
        ("qo_indptr", ctypes.c_void_p),
        ("qo_indptr_host", ctypes.c_void_p),
        ("logits_soft_cap", ctypes.c_float),
        ("merge_mode", ctypes.c_int32),
        ("wave_split", ctypes.c_int32),
    ]


class KvsPlanInfo(ctypes.Structure):
    _fields_ = [
        ("kv_chunk", ctypes.c_int32),
        ("items_per_kv_head", ctypes.c_int32),
        ("max_splits", ctypes.c_int32),
        ("needs_merge", ctypes.c_int32),
        ("algo", ctypes.c_int32),
        ("num_cus", ctypes.c_int32),
        ("workspace_bytes", ctypes.c_size_t),
        ("col_groups", ctypes.c_int32),
        ("col_share", ctypes.c_int32),
        ("merge_in_partial", ctypes.c_int32),
        ("wave_packs", ctypes.c_int32),
        ("part_format", ctypes.c_int32),
    ]


class KvsAppendArgs(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("num_qo_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("q_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("num_pages", ctypes.c_int32),
        ("q_in", ctypes.c_void_p),
        ("k_in", ctypes.c_void_p),
        ("v_in", ctypes.c_void_p),
        ("q_out", ctypes.c_void_p),
        ("k_cache", ctypes.c_void_p),
        ("v_cache", ctypes.c_void_p),
        ("page_indptr", ctypes.c_void_p),
        ("page_indices", ctypes.c_void_p),
        ("kv_len", ctypes.c_void_p),
        ("k_scale", ctypes.c_void_p),
        ("v_scale", ctypes.c_void_p),
        ("q_norm_weight", ctypes.c_void_p),
        ("k_norm_weight", ctypes.c_void_p),
        ("norm_eps", ctypes.c_float),
        ("rope_theta", ctypes.c_float),
        ("rope_interleave", ctypes.c_int32),
        ("prof_events", ctypes.c_void_p * 2),
        ("qo_indptr", ctypes.c_void_p),
        ("qo_indptr_host", ctypes.c_void_p),
    ]


class KvsError(RuntimeError):
    def __init__(self, status: int, what: str = "kvs_decode"):
        self.status = status
        super().__init__(f"{what}: {kvs_status_string(status)} (status {status})")


_lib = None
_lib_lock = threading.Lock()


def load_library():
    """Load libkvsplit.so; raises if it has not been built."""
    global _lib
    with _lib_lock:
        if _lib is None:
            path = library_path()
            if not os.path.exists(path):
                raise RuntimeError(
                    f"libkvsplit.so is not built ({path}); run `python -m decode_attention_kv_split_amd.build`")
            lib = ctypes.CDLL(path)
            lib.kvs_decode.restype = ctypes.c_int
            lib.kvs_decode.argtypes = [ctypes.POINTER(KvsDecodeArgs), ctypes.c_void_p, ctypes.c_size_t,
                                       ctypes.c_void_p]
            lib.kvs_decode_noalloc.restype = ctypes.c_int
            lib.kvs_decode_noalloc.argtypes = [ctypes.POINTER(KvsDecodeArgs), ctypes.c_void_p]
            lib.kvs_decode_plan.restype = ctypes.c_int
            lib.kvs_decode_plan.argtypes = [ctypes.POINTER(KvsDecodeArgs), ctypes.POINTER(KvsPlanInfo)]
            lib.kvs_decode_workspace_bytes.restype = ctypes.c_size_t
            lib.kvs_decode_workspace_bytes.argtypes = [ctypes.POINTER(KvsDecodeArgs)]
            lib.kvs_append.restype = ctypes.c_int
            lib.kvs_append.argtypes = [ctypes.POINTER(KvsAppendArgs), ctypes.c_void_p]
            lib.kvs_status_string.restype = ctypes.c_char_p
            lib.kvs_status_string.argtypes = [ctypes.c_int]
            lib.kvs_abi_version.restype = ctypes.c_int
            lib.kvs_abi_version.argtypes = []
            lib.kvs_probe_stream_read.restype = ctypes.c_int
            lib.kvs_probe_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                                  ctypes.c_void_p]
            lib.kvs_probe_copy.restype = ctypes.c_int
            lib.kvs_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
            _lib = lib
    return _lib


# ----------------------------------------------------------------------------
# C ABI, same names
# ----------------------------------------------------------------------------

def kvs_decode(args: KvsDecodeArgs, workspace: int, workspace_bytes: int, stream: int) -> int:
    return int(load_library().kvs_decode(ctypes.byref(args), ctypes.c_void_p(workspace or None),
                                         ctypes.c_size_t(workspace_bytes), ctypes.c_void_p(stream or None)))


def kvs_decode_noalloc(args: KvsDecodeArgs, stream: int) -> int:
    return int(load_library().kvs_decode_noalloc(ctypes.byref(args), ctypes.c_void_p(stream or None)))


def kvs_decode_plan(args: KvsDecodeArgs) -> KvsPlanInfo:
    info = KvsPlanInfo()
    st = int(load_library().kvs_decode_plan(ctypes.byref(args), ctypes.byref(info)))
    if st != KVS_OK:
        raise KvsError(st, "kvs_decode_plan")
    return info


def kvs_decode_workspace_bytes(args: KvsDecodeArgs) -> int:
    return int(load_library().kvs_decode_workspace_bytes(ctypes.byref(args)))


def kvs_append(args: KvsAppendArgs, stream: int) -> int:
    return int(load_library().kvs_append(ctypes.byref(args), ctypes.c_void_p(stream or None)))


def kvs_status_string(status: int) -> str:
    return load_library().kvs_status_string(int(status)).decode()


def kvs_abi_version() -> int:
    return int(load_library().kvs_abi_version())


def kvs_probe_stream_read(buf_ptr: int, nbytes: int, sink_ptr: int, stream: int) -> int:
    return int(load_library().kvs_probe_stream_read(ctypes.c_void_p(buf_ptr), ctypes.c_size_t(nbytes),
                                                    ctypes.c_void_p(sink_ptr or None),
                                                    ctypes.c_void_p(stream or None)))


def kvs_probe_copy(dst_ptr: int, src_ptr: int, nbytes: int, stream: int) -> int:
    return int(load_library().kvs_probe_copy(ctypes.c_void_p(dst_ptr), ctypes.c_void_p(src_ptr),
                                             ctypes.c_size_t(nbytes), ctypes.c_void_p(stream or None)))


# ----------------------------------------------------------------------------
# torch marshalling
# ----------------------------------------------------------------------------

_KV_NAMES = {"f32": KVS_F32, "bf16": KVS_BF16, "fp8": KVS_FP8_E4M3, "int4": KVS_INT4}


def _dtype_code(t, what: str, name: Optional[str] = None) -> int:
    """kvs_dtype of a tensor; ``name`` ('f32', 'bf16', 'fp8', 'int4') settles
    byte tensors, which hold fp8 codes unless told they are packed INT4."""
    import torch

    if name is not None:
        return _KV_NAMES[name]
    if t.dtype == torch.float32:
        return KVS_F32
    if t.dtype == torch.bfloat16:
        return KVS_BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8) and what == "kv":
        return KVS_FP8_E4M3
    raise ValueError(f"unsupported {what} dtype {t.dtype}")


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _check_dev(t, name: str, device) -> None:
    if t is None:
        return
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_ws_cache = {}
_ws_lock = threading.Lock()


def _workspace(nbytes: int, device, stream: int):
    """Per (device, stream) scratch buffer, grown on demand (torch allocation).

    The buffer is allocated on the stream that uses it, so that when a larger
    one replaces it, torch's caching allocator hands its memory out again
    only in that stream's order (after the kernels that still use it)."""
    import torch

    if nbytes == 0:
        return None
    key = (device.index, stream)
    with _ws_lock:
        buf = _ws_cache.get(key)
        if buf is None or buf.numel() < nbytes:
            # zeroed: the first KVS_WORKSPACE_COUNTER_BYTES are merge counters
            # that must start at zero (every call leaves them zero)
            with torch.cuda.device(device), torch.cuda.stream(torch.cuda.ExternalStream(stream, device=device)):
                buf = torch.zeros(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            _ws_cache[key] = buf
    return buf


def make_args(q, k, v, kv_len, *, page_indptr=None, page_indices=None, kv_len_host=None,
              k_scale=None, v_scale=None, sm_scale=None, window: int = -1, kv_chunk: int = 0,
              algo="auto", out=None, lse=None, num_cus: int = 0,
              unified_max: Optional[float] = None, kv_dtype: Optional[str] = None, qo_indptr=None,
              qo_indptr_host=None, logits_soft_cap: float = 0.0,
              merge_mode="auto", wave_split="auto") -> Tuple[KvsDecodeArgs, object]:
    """Build the C argument block from torch tensors.

    q: [batch, Hq, d]; k, v: contiguous [kv_len, Hk, d] (batch 1) or paged
    [num_pages, page_size, Hk, d]; kv_len: int32 [batch] on the device.
    kv_dtype='int4' marks uint8 caches whose last axis holds d / 2 bytes of
    packed nibbles.  qo_indptr (int32 [batch + 1] on the device, with a host
    copy) gives several query rows per request: q is then [total_q, Hq, d].
    logits_soft_cap c > 0 caps the scaled scores to c * tanh(s / c).
    merge_mode: "auto" | "in_partial" | "kernel"; wave_split: "auto" |
    "heads" | "tiles" (how a matrix-core workgroup's waves share its work).
    Returns (args, keepalive)."""
    import numpy as np
    import torch

    device = q.device
    if q.dim() != 3:
        raise ValueError("q must be [batch (or total_q), num_qo_heads, head_dim]")
    rows, Hq, d = q.shape
    B = int(kv_len.numel())
    qoh = None
    if qo_indptr is not None:
        src = qo_indptr_host if qo_indptr_host is not None else qo_indptr.cpu()
        qoh = np.ascontiguousarray(np.asarray(src.cpu() if isinstance(src, torch.Tensor) else src, dtype=np.int32))
        if qoh.shape != (B + 1,) or int(qoh[-1]) != rows:
            raise ValueError("qo_indptr must be [batch + 1] ending at q's row count")
        if qo_indptr.dtype != torch.int32 or qo_indptr.numel() != B + 1:
            raise ValueError("qo_indptr must be int32 [batch + 1]")
    elif rows != B:
        raise ValueError("q must have one row per request without qo_indptr")
    paged = page_indptr is not None
    if paged:
        if k.dim() != 4:
            raise ValueError("paged k/v must be [num_pages, page_size, num_kv_heads, head_dim]")
        num_pages, P, Hk, dk = k.shape
    else:
        if k.dim() != 3:
            raise ValueError("contiguous k/v must be [kv_len, num_kv_heads, head_dim]")
        capacity, Hk, dk = k.shape
        P, num_pages = 0, capacity
    if v.shape != k.shape or v.dtype != k.dtype:
        raise ValueError("k and v must have the same shape and dtype")
    if kv_dtype == "int4":
        if k.dtype != torch.uint8 or 2 * dk != d:
            raise ValueError("int4 k/v must be uint8 with head_dim / 2 bytes per row")
    elif dk != d:
        raise ValueError("head_dim of q and k differ")
    if kv_len.dtype != torch.int32 or kv_len.numel() != B:
        raise ValueError("kv_len must be int32 [batch]")
    if kv_len_host is None:
        kv_len_host = kv_len.cpu()
    kvh = np.ascontiguousarray(np.asarray(kv_len_host.cpu() if isinstance(kv_len_host, torch.Tensor)
                                          else kv_len_host, dtype=np.int32))
    if kvh.shape != (B,):
        raise ValueError("kv_len_host must hold one length per request")
    if not paged and B and int(kvh.max()) > k.shape[0]:
        raise ValueError("kv_len exceeds the rows of the contiguous cache")
    if out is None:
        out = torch.empty((rows, Hq, d), dtype=q.dtype, device=device)
    elif tuple(out.shape) != (rows, Hq, d) or out.dtype != q.dtype:
        raise ValueError(f"out must be [{rows}, {Hq}, {d}] in q's dtype")
    if lse is None:
        lse = torch.empty((rows, Hq), dtype=torch.float32, device=device)
    elif tuple(lse.shape) != (rows, Hq) or lse.dtype != torch.float32:
        raise ValueError(f"lse must be float32 [{rows}, {Hq}]")
    # shapes and types first (above), then where the tensors live
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (kv_len, "kv_len"), (page_indptr, "page_indptr"),
                 (page_indices, "page_indices"), (k_scale, "k_scale"), (v_scale, "v_scale"),
                 (qo_indptr, "qo_indptr"), (out, "out"), (lse, "lse")):
        _check_dev(t, n, device)
    a = KvsDecodeArgs()
    a.batch, a.num_qo_heads, a.num_kv_heads, a.head_dim = B, Hq, Hk, d
    a.q_dtype = _dtype_code(q, "q")
    a.kv_dtype = _dtype_code(k, "kv", kv_dtype)
    a.page_size, a.num_pages = P, num_pages
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.page_indptr, a.page_indices = _ptr(page_indptr), _ptr(page_indices)
    a.kv_len = _ptr(kv_len)
    a.kv_len_host = kvh.ctypes.data
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.sm_scale = float(1.0 / math.sqrt(d) if sm_scale is None else sm_scale)
    a.window = int(window)
    a.kv_chunk = int(kv_chunk)
    a.algo = _ALGOS[algo] if isinstance(algo, str) else int(algo)
    a.num_cus = int(num_cus)
    a.o, a.lse = _ptr(out), _ptr(lse)
    if unified_max is not None:
        a.use_unified_max, a.unified_max = 1, float(unified_max)
    if qoh is not None:
        a.qo_indptr, a.qo_indptr_host = _ptr(qo_indptr), qoh.ctypes.data
    a.logits_soft_cap = float(logits_soft_cap)
    a.merge_mode = _MERGE_MODES[merge_mode] if isinstance(merge_mode, str) else int(merge_mode)
    a.wave_split = _WAVE_SPLITS[wave_split] if isinstance(wave_split, str) else int(wave_split)
    keep = (kvh, out, lse, qoh)
    return a, keep


def decode(q, k, v, kv_len, *, page_indptr=None, page_indices=None, kv_len_host=None, k_scale=None,
           v_scale=None, sm_scale=None, window: int = -1, kv_chunk: int = 0, algo="auto", out=None, lse=None,
           workspace=None, stream=None, unified_max: Optional[float] = None, kv_dtype: Optional[str] = None,
           qo_indptr=None, qo_indptr_host=None, logits_soft_cap: float = 0.0, merge_mode="auto",
           wave_split="auto", num_cus: int = 0):
    """One decode-attention step on the current (or given) HIP stream.
    num_cus: CU count to plan for (0: the device's).
    Returns (o [batch, Hq, d] in q's dtype, lse [batch, Hq] fp32, natural log)."""
    import torch

    a, keep = make_args(q, k, v, kv_len, page_indptr=page_indptr, page_indices=page_indices,
                        kv_len_host=kv_len_host, k_scale=k_scale, v_scale=v_scale, sm_scale=sm_scale,
                        window=window, kv_chunk=kv_chunk, algo=algo, out=out, lse=lse, unified_max=unified_max,
                        kv_dtype=kv_dtype, qo_indptr=qo_indptr, qo_indptr_host=qo_indptr_host,
                        logits_soft_cap=logits_soft_cap, merge_mode=merge_mode, wave_split=wave_split,
                        num_cus=num_cus)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else int(stream)
    need = kvs_decode_workspace_bytes(a)
    if workspace is None:
        ws = _workspace(need, q.device, s)
        ws_ptr, ws_bytes = (ws.data_ptr(), ws.numel()) if ws is not None else (0, 0)
    else:
        ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    st = kvs_decode(a, ws_ptr, ws_bytes, s)
    if st != KVS_OK:
        if st in (KVS_ERR_INVALID_ARG, KVS_ERR_UNSUPPORTED, KVS_ERR_WORKSPACE):
            raise ValueError(f"kvs_decode: {kvs_status_string(st)}")
        raise KvsError(st)
    return keep[1], keep[2]


def single_decode(q, k, v, *, sm_scale=None, window: int = -1, kv_chunk: int = 0, algo="auto",
                  k_scale=None, v_scale=None):
    """One request: q [Hq, d], k/v [kv_len, Hk, d].  Returns (o [Hq, d], lse [Hq])."""
    import torch

    L = k.shape[0]
    kv_len = torch.tensor([L], dtype=torch.int32, device=q.device)
    o, lse = decode(q[None], k, v, kv_len, kv_len_host=[L], sm_scale=sm_scale, window=window,
                    kv_chunk=kv_chunk, algo=algo, k_scale=k_scale, v_scale=v_scale)
    return o[0], lse[0]


def batch_decode_paged(q, k_pages, v_pages, page_indptr, page_indices, kv_len, *, kv_len_host=None,
                       sm_scale=None, window: int = -1, kv_chunk: int = 0, algo="auto", k_scale=None,
                       v_scale=None):
    """Batched decode over a paged cache; q [batch, Hq, d]."""
    return decode(q, k_pages, v_pages, kv_len, page_indptr=page_indptr, page_indices=page_indices,
                  kv_len_host=kv_len_host, sm_scale=sm_scale, window=window, kv_chunk=kv_chunk, algo=algo,
                  k_scale=k_scale, v_scale=v_scale)


def make_append_args(q, k, v, k_cache, v_cache, kv_len, *, page_indptr=None, page_indices=None,
                     k_scale=None, v_scale=None, q_norm_weight=None, k_norm_weight=None,
                     norm_eps: float = 1e-6, rope_theta: float = 10000.0, rope_interleave: bool = False,
                     q_out=None, qo_indptr=None, qo_indptr_host=None,
                     kv_dtype: Optional[str] = None) -> Tuple[KvsAppendArgs, object]:
    """Build the C argument block of kvs_append from torch tensors.

    q [rows, Hq, d], k and v [rows, Hk, d] (q's dtype), rows = batch (one new
    token per request) or qo_indptr[batch] (qo_indptr: int32 [batch + 1] on
    the device, with a host copy; request b's rows are qo_indptr[b] ..
    qo_indptr[b+1] - 1, row i at position kv_len[b] + i).  The cache as for
    decode (paged [num_pages, page_size, Hk, d] or contiguous
    [capacity, Hk, d]; kv_dtype='int4' marks uint8 caches of d / 2 packed
    bytes per row); kv_len int32 [batch] on the device (tokens cached
    before the call).  q_out defaults to a new tensor; it may be q."""
    import numpy as np
    import torch

    device = q.device
    rows, Hq, d = q.shape
    B = int(kv_len.numel())
    Hk = k.shape[1]
    if k.shape != (rows, Hk, d) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [rows, num_kv_heads, head_dim] in q's dtype")
    qoh = None
    if qo_indptr is not None:
        src = qo_indptr_host if qo_indptr_host is not None else qo_indptr.cpu()
        qoh = np.ascontiguousarray(np.asarray(src.cpu() if isinstance(src, torch.Tensor) else src, dtype=np.int32))
        if qoh.shape != (B + 1,) or int(qoh[-1]) != rows or int(qoh[0]) != 0 or np.any(np.diff(qoh) < 0):
            raise ValueError("qo_indptr must be [batch + 1], non-decreasing from 0 to q's row count")
        if qo_indptr.dtype != torch.int32 or qo_indptr.numel() != B + 1:
            raise ValueError("qo_indptr must be int32 [batch + 1]")
    elif rows != B:
        raise ValueError("q must have one row per request without qo_indptr")
    paged = page_indptr is not None
    if paged:
        num_pages, P, Hk2, d2 = k_cache.shape
    else:
        num_pages, Hk2, d2 = k_cache.shape
        P = 0
    int4 = kv_dtype == "int4"
    if int4 and k_cache.dtype != torch.uint8:
        raise ValueError("an int4 cache is uint8 with head_dim / 2 bytes per row")
    if (Hk2, d2) != (Hk, d // 2 if int4 else d) or v_cache.shape != k_cache.shape or v_cache.dtype != k_cache.dtype:
        raise ValueError("cache shape does not match the new tokens")
    if kv_len.dtype != torch.int32 or kv_len.numel() != B:
        raise ValueError("kv_len must be int32 [batch]")
    if q_out is None:
        q_out = torch.empty_like(q)
    elif q_out.shape != q.shape or q_out.dtype != q.dtype:
        raise ValueError("q_out must have q's shape and dtype")
    for w, n in ((q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight")):
        if w is not None and (w.dtype != torch.float32 or w.numel() != d):
            raise ValueError(f"{n} must be float32 [head_dim]")
    for t, n in ((q, "q"), (k, "k"), (v, "v"), (k_cache, "k_cache"), (v_cache, "v_cache"), (kv_len, "kv_len"),
                 (page_indptr, "page_indptr"), (page_indices, "page_indices"), (k_scale, "k_scale"),
                 (v_scale, "v_scale"), (q_norm_weight, "q_norm_weight"), (k_norm_weight, "k_norm_weight"),
                 (q_out, "q_out"), (qo_indptr, "qo_indptr")):
        _check_dev(t, n, device)
    a = KvsAppendArgs()
    a.batch, a.num_qo_heads, a.num_kv_heads, a.head_dim = B, Hq, Hk, d
    a.q_dtype = _dtype_code(q, "q")
    a.kv_dtype = _dtype_code(k_cache, "kv", kv_dtype)
    a.page_size, a.num_pages = P, num_pages
    a.q_in, a.k_in, a.v_in, a.q_out = _ptr(q), _ptr(k), _ptr(v), _ptr(q_out)
    a.k_cache, a.v_cache = _ptr(k_cache), _ptr(v_cache)
    a.page_indptr, a.page_indices = _ptr(page_indptr), _ptr(page_indices)
    a.kv_len = _ptr(kv_len)
    a.k_scale, a.v_scale = _ptr(k_scale), _ptr(v_scale)
    a.q_norm_weight, a.k_norm_weight = _ptr(q_norm_weight), _ptr(k_norm_weight)
    a.norm_eps = float(norm_eps)
    a.rope_theta = float(rope_theta)
    a.rope_interleave = int(bool(rope_interleave))
    if qoh is not None:
        a.qo_indptr, a.qo_indptr_host = _ptr(qo_indptr), qoh.ctypes.data
    return a, (q_out, qoh)


def append(q, k, v, k_cache, v_cache, kv_len, *, page_indptr=None, page_indices=None, k_scale=None,
           v_scale=None, q_norm_weight=None, k_norm_weight=None, norm_eps: float = 1e-6,
           rope_theta: float = 10000.0, rope_interleave: bool = False, q_out=None, stream=None,
           qo_indptr=None, qo_indptr_host=None, kv_dtype: Optional[str] = None):
    """QK-norm and rotary embedding of the new tokens, and their K/V stored
    after each request's cached tokens (one per request at kv_len[b], or the
    rows of qo_indptr at kv_len[b] + i).  Returns q_out.  kv_len is not
    changed."""
    import torch

    a, keep = make_append_args(q, k, v, k_cache, v_cache, kv_len, page_indptr=page_indptr,
                               page_indices=page_indices, k_scale=k_scale, v_scale=v_scale,
                               q_norm_weight=q_norm_weight, k_norm_weight=k_norm_weight, norm_eps=norm_eps,
                               rope_theta=rope_theta, rope_interleave=rope_interleave, q_out=q_out,
                               qo_indptr=qo_indptr, qo_indptr_host=qo_indptr_host, kv_dtype=kv_dtype)
    s = torch.cuda.current_stream(q.device).cuda_stream if stream is None else int(stream)
    st = kvs_append(a, s)
    if st != KVS_OK:
        if st in (KVS_ERR_INVALID_ARG, KVS_ERR_UNSUPPORTED):
            raise ValueError(f"kvs_append: {kvs_status_string(st)}")
        raise KvsError(st, "kvs_append")
    return keep[0]
