"""CPU oracle for routed FP16/INT8 prefill attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product library or its binding.
"""
from .tilemix_oracle import *  # noqa: F401,F403
from .tilemix_oracle import (AttnInputs, attn_prefill, attn_rows, attn_tile_row, attn_dense_two_pass,
                             attn_brute_force, build_route_mask, decode_route_mask, quantize_blockwise,
                             route_bit, route_used, s32_tiles, visit_matrix, footprint_bytes,
                             qk_tile_operand_bytes, nearest_fp32, num_tiles, seq_spans)
