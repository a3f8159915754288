"""Seeded synthetic inputs for the QSA decode path.

This package holds only random-number generation and storage encoding of
inputs (BF16 / FP8 bit patterns), plus the re-layout of a workload's KV
caches into randomly placed pages.  It contains none of the method's
arithmetic (no scoring, selection, position building or attention), so both
the CPU oracle's tests and the GPU path can draw identical bytes from it.
"""
from .gen import (CONFIGS, Workload, make_workload, make_custom, bf16_bits_from_f32,
                  fp8_e4m3fn_bits_from_f32, normal_quantile_table, paged_layout)

__all__ = ["CONFIGS", "Workload", "make_workload", "make_custom", "bf16_bits_from_f32",
           "fp8_e4m3fn_bits_from_f32", "normal_quantile_table", "paged_layout"]
