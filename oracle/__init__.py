"""CPU oracle for ExpCast FP8 attention (float64 numpy).

TEST INFRASTRUCTURE ONLY. It may be imported by tests/, by the smoke check in
__graft_entry__.py and by the CPU-baseline leg of bench.py, and by nothing
else. It shares no code, table or constant generator with the GPU library
under bit_fp8_attention_block_amd/, and neither side imports the other.

Pins (tests/test_oracle_*.py) tie it to facts fixed by the pages and by the
mathematics: the E4M3 format definition and a library cast, the byte/log2
relation of the VC-Attention write-up, the 79.6% agreement and 3.64%
total-variation figures of its "ExpCast-FP8" section (reproduced from closed
forms), brute force on tiny inputs, and special cases with closed-form
outputs. Every function is pinned; none is marked "parity unpinned".
"""
from .e4m3 import E4M3_MAX, VALUES, decode, encode  # noqa: F401
from .expcast import (  # noqa: F401
    BETA, CODE_OF_PMAX, QK_BLOCK, PreparedHead, RepairSet, bitaligned_row_max,
    exact_attention_head, exp_cast_codes, expcast_attention_head, expcast_attention_online, expcast_codes,
    key_mean, key_tile_order, smooth_keys, smooth_values, to_bf16, value_block_means,
    log2_logits, prepare_head, quant_scale, quantize_blocks, quantize_head, residual_energy, SCALE_FLOOR,
    quantize_with, rel_l2, repair_count, repair_select, row_total_variation,
)
