"""Seeded synthetic inputs for the sparse-attention indexer (scoring + exact top-k).

This package only draws random numbers and lays them out in the index-cache
format; it holds none of the scoring or selection arithmetic. Both the CPU
oracle and the GPU path read what it produces.
"""
from .synth import Problem, make_config, make_problem, rope_table, CONFIG_NAMES, FULL_CONFIGS

__all__ = ["Problem", "make_config", "make_problem", "rope_table", "CONFIG_NAMES", "FULL_CONFIGS"]
