"""Oracle for split-KV decode attention and the step before it (QK-norm,
rotary embedding, KV append): plain, slow, obviously correct, fp64.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no
code with the HIP library (``decode_attention_kv_split_amd``), which never
imports it; the product path has no CPU fallback.

Every function is pinned by the CPU tests against closed forms, brute
force (``math.fsum`` / ``decimal``), library routines (torch's casts for
the codecs) and invariants of the definition; see ``tests/test_oracle.py``,
``tests/test_codecs.py`` and ``tests/test_append_oracle.py``.
"""
from .append import (append_codes, append_reference, apply_append, cache_slot, rms_norm, rope,
                     rope_angles, token_rows, transform_head)
from .codecs import (bf16_to_f64, decode_codes, encode_codes, f64_to_bf16_codes, f64_to_fp8_e4m3fn_codes,
                     f64_to_int4_codes, fp8_e4m3fn_to_f64, int4_to_f64, round_to_grid)
from .multi import attention_reference, query_position, query_range
from .decode import (attend_chunked, attend_direct, cap_scores, chunk_state, decode_reference,
                     decode_reference_chunked, decode_reference_sampled, kv_head_of,
                     merge_states, request_kv, softmax_from_scores, visible_range)

__all__ = [
    "bf16_to_f64", "fp8_e4m3fn_to_f64", "int4_to_f64", "decode_codes", "encode_codes", "f64_to_bf16_codes",
    "f64_to_fp8_e4m3fn_codes", "f64_to_int4_codes", "round_to_grid",
    "rms_norm", "rope", "rope_angles", "transform_head", "append_reference", "append_codes",
    "apply_append", "cache_slot", "token_rows",
    "attend_direct", "attend_chunked", "cap_scores", "chunk_state", "merge_states", "softmax_from_scores",
    "decode_reference", "decode_reference_chunked", "decode_reference_sampled",
    "kv_head_of", "visible_range", "request_kv",
    "attention_reference", "query_position", "query_range",
]
