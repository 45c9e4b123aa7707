"""CPU oracle of the block-wise mixed-precision quantized matmul.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and the cpu_baseline
leg of bench.py may import it.  The library never does.
"""
from .msq_oracle import *  # noqa: F401,F403
from .msq_oracle import (ALLOWED_BITS, BLOCK_COLS, BLOCK_ROWS, NO_BLOCK, SEGMENT_ORDER,  # noqa: F401
                         bf16_to_f32, block_offsets, dequantize, group_params, matmul, pack,
                         pack_blocks, quantize, quantize_codes, quantize_pack, reference_gemm,
                         reorder, unpack, unpack_blocks, validate)
