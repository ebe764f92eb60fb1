"""Seeded synthetic inputs shared by the tests and the bench.

This package draws random numbers and lays them out in the stored formats
(bf16, e4m3, packed FP8 latent rows, pages).  It contains none of the
method's arithmetic: no score, no selection, no attention.  Both the CPU
oracle (through host copies) and the HIP library consume what it makes.
"""
from .gen import (CONFIGS, Call, Inputs, Workload, config, generate,
                  lognormal_context_lengths)

__all__ = ["CONFIGS", "Call", "Inputs", "Workload", "config", "generate",
           "lognormal_context_lengths"]
