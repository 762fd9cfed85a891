"""CPU oracle for TileMix prefill, INT8-cache decode attention and the synthetic
multi-layer stack (test infrastructure only: used by tests/,
__graft_entry__.smoke() and bench.py's cpu_baseline leg)."""
from .tilemix_oracle import *  # noqa: F401,F403
from .tilemix_oracle import (BLOCK_M, BLOCK_N, TEMPLATES, SeqGeometry, seq_geometry,  # noqa: F401
                             int8_group_count, template_order, int8_groups, routing_words,
                             quantize_blocks, qk_int32_tile, prefill_attention, run,
                             splitmix64_mix, rowrandom_hash, sptrans_stride, union_orders,
                             softmax_scale, int8_tile_scale, quantize_kv_cache,
                             quantize_query_rows, decode_attention, block_column_sums,
                             routing_importance, adaptive_words, importance_exposure, FP8_MAX,
                             fp8_e4m3_decode, fp8_e4m3_encode, quantize_blocks_fp8, routing_words3,
                             prefill_attention3, STACK_EPS, stack_width, stack_rms_norm,
                             stack_qkv, stack_out_residual, stack_layer, stack_forward,
                             depth_deviation)
