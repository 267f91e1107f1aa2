"""Seeded synthetic layer workloads shared by the tests, the oracle runs and
the benchmark. Holds random draws and dtype rounding only: none of the
quantization method's arithmetic lives here."""
from .workloads import (RECIPES, Workload, bf16_bits_to_f32, f32_to_bf16_bits,
                        make_workload, gen_W, iter_X, x_full)

__all__ = ["RECIPES", "Workload", "bf16_bits_to_f32", "f32_to_bf16_bits",
           "make_workload", "gen_W", "iter_X", "x_full"]
