"""CPU oracle (test infrastructure only: tests, smoke check, CPU baseline).

The GPU product path never imports this package.
"""
from .q3_oracle import *  # noqa: F401,F403
from .q3_oracle import (E4M3FN_TABLE, bf16_decode, dequantize, e4m3fn_decode, e8m0_decode, word_offset, scale_offset,  # noqa: F401,E501
                        expert_union, grouped_linear, layout, linear, pack, pack_group,
                        topk_route, unpack, unpack_group, within_tolerance, budget_route, routing_mass,
                        combine_weights, moe_mlp, silu)
from .q2_head import (decide, dequantize2, layout2, linear2, mxfp8_dequantize, pack2, pack_group2,  # noqa: F401
                      rescore, shortlist, unpack2, unpack_group2, word_offset2)
from .q3_quant import choose_scales, codebook_values, quantize, snap  # noqa: F401,E402
from .q3_fit import fit_codebook, fit_row, grid_values, group_exponents, lloyd, round_e4m3fn  # noqa: F401,E402
