"""MI355X-native FlashAttention-2 forward (bf16, fp32 and FP8-e4m3).

The compute runs in hand-written gfx950 HIP kernels behind the C ABI declared
in include/fa.h (libfa.so). This package is the thin Python binding over that
library; torch is used only for device memory and streams.
"""
from .inputs import WORKLOADS, Workload, make_qkv, make_workload, sample_rows  # noqa: F401
