"""3-bit FP8-codebook decode linear layers for MI355X (gfx950).

Thin Python binding over libq3.so (include/q3.h).  Build the library with
`python -m bit_fp8_codebook_amd.build`; importing the ops without it raises.
"""
from ._lib import (ExpertStack, Mxfp8Head, PackedHead2, PackedMatrix, Q3Error, draft_head_workspace,  # noqa: F401
                   empty_packed, empty_stack, lib, moe_mlp_workspace, q3_draft_head, q3_fit_codebook, q3_gemm_small_m,
                   q3_gemm_small_m_workspace_bytes, q3_gemm_small_m_ws, q3_gemv, q3_grouped_expert_gemv,
                   q3_head2_scores, q3_layout, q3_layout2, q3_moe_budget_topk, q3_moe_mlp, q3_moe_mlp_noalloc,
                   q3_moe_mlp_noalloc_max_bytes, q3_moe_topk, q3_pack,
                   q3_pack2, q3_quantize, q3_rescore_fp8, q3_shortlist, q3_unpack, q3_unpack2)
