"""Seeded synthetic inputs for the LoopVQ hot path.

This package is the only code shared by the CPU oracle and the HIP path: it
draws inputs (loop-correlated K/V caches, queries, sinks, channel weights and
permutations, calibration codebooks) and nothing else.  Neither side's
results are computed here.
"""
from .configs import CONFIGS, LoopConfig, config_by_index
from .generator import (SeedPlan, gen_kv_layer, gen_queries, gen_sinks,
                        gen_tasq_params, gen_calibration_kv)
from .codebooks import train_codebooks
from .inputs import build_inputs, random_codebooks
from .toy import gen_targets, gen_toy_stack

__all__ = ["CONFIGS", "LoopConfig", "config_by_index", "SeedPlan",
           "gen_kv_layer", "gen_queries", "gen_sinks", "gen_tasq_params",
           "gen_calibration_kv", "train_codebooks", "build_inputs",
           "random_codebooks", "gen_toy_stack", "gen_targets"]
