"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

Inputs only: nothing in this package computes any part of the recall method.
"""
from .synth import (CONFIG_NAMES, CONFIG_SEEDS, DEFAULT_A1, DEFAULT_A2,
                    DEFAULT_AFP, DEFAULT_L, DEFAULT_R, GENERATORS, Workload,
                    fill_random_bytes, gen_fuzz, gen_medium, make)

__all__ = ["CONFIG_NAMES", "CONFIG_SEEDS", "DEFAULT_A1", "DEFAULT_A2",
           "DEFAULT_AFP", "DEFAULT_L", "DEFAULT_R", "GENERATORS", "Workload",
           "fill_random_bytes", "gen_fuzz", "gen_medium", "make"]
