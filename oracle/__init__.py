"""Oracle for split-KV decode attention: plain, slow, obviously correct, fp64.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``decode_attention_kv_split_amd``), which never
imports it; the product path has no CPU fallback.

Every function is pinned by the CPU tests against closed forms, brute
force (``math.fsum`` / ``decimal``), library routines (torch's casts for
the codecs) and invariants of the definition; see ``tests/test_oracle.py``.
"""
from .codecs import bf16_to_f64, decode_codes, fp8_e4m3fn_to_f64
from .decode import (attend_chunked, attend_direct, chunk_state, decode_reference,
                     decode_reference_chunked, decode_reference_sampled, kv_head_of,
                     merge_states, request_kv, softmax_from_scores, visible_range)

__all__ = [
    "bf16_to_f64", "fp8_e4m3fn_to_f64", "decode_codes",
    "attend_direct", "attend_chunked", "chunk_state", "merge_states", "softmax_from_scores",
    "decode_reference", "decode_reference_chunked", "decode_reference_sampled",
    "kv_head_of", "visible_range", "request_kv",
]
