"""CPU oracle for QSA block-sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  The library path never calls it, and it
shares no code with the HIP kernels.
"""
from .qsa_oracle import (BLOCK, TOPK, WIDTH, bf16_to_f64, fp8_e4m3fn_to_f64, query_length,
                         block_scores, select_blocks, build_positions, sparse_attention,
                         decode)

__all__ = ["BLOCK", "TOPK", "WIDTH", "bf16_to_f64", "fp8_e4m3fn_to_f64", "query_length",
           "block_scores", "select_blocks", "build_positions", "sparse_attention", "decode"]
