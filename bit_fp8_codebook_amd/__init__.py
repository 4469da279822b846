"""3-bit FP8-codebook decode linear layers for MI355X (gfx950).

Thin Python binding over libq3.so (include/q3.h).  Build the library with
`python -m bit_fp8_codebook_amd.build`; importing the ops without it raises.
"""
from ._lib import (ExpertStack, PackedMatrix, Q3Error, empty_packed, empty_stack, lib,  # noqa: F401
                   q3_gemm_small_m, q3_gemv, q3_grouped_expert_gemv, q3_layout, q3_moe_topk, q3_pack,
                   q3_unpack)
