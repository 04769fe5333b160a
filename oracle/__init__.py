"""fp64 CPU oracle for the FlashAttention-2 forward, its split-KV partials and
their merge, grouped-query attention, the backward pass, the per-head FP8
quantiser, the rotation applied before it and per-block (microscaled) FP8. TEST INFRASTRUCTURE ONLY: imported by tests/, by
__graft_entry__.smoke() and by bench.py's cpu_baseline leg, never by the
product path. It shares no code with the HIP library."""
from .attention import attention, attention_online, attention_bruteforce  # noqa: F401
from .splitkv import attention_keyrange, merge_partials  # noqa: F401
from .gqa import attention_gqa, kv_head_of  # noqa: F401
from .backward import attention_backward, attention_backward_rows  # noqa: F401
from .rotation import hadamard, rotate, quantize_rotated  # noqa: F401
from .fp8 import (e4m3_table, e4m3_encode, e4m3_decode, quantize_per_head,  # noqa: F401
                  dequantize_per_head, E4M3_MAX)
from .mxfp8 import mx_exponent, quantize_mx, dequantize_mx, quantize_qkv_mx, quantize_rotated_mx  # noqa: F401
