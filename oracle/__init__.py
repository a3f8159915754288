"""CPU oracle for QSA block-sparse decode attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  The library path never calls it, and it
shares no code with the HIP kernels.
"""
from .qsa_oracle import (BLOCK, TOPK, WIDTH, bf16_to_f64, fp8_e4m3fn_to_f64, query_length,
                         block_scores, select_blocks, token_slots, build_positions, sparse_attention,
                         bf16_bits_round_exact, compress_block_key, compress_new_keys, decode)

__all__ = ["BLOCK", "TOPK", "WIDTH", "bf16_to_f64", "fp8_e4m3fn_to_f64", "query_length",
           "block_scores", "select_blocks", "token_slots", "build_positions", "sparse_attention",
           "bf16_bits_round_exact", "compress_block_key", "compress_new_keys", "decode"]
