"""Seeded synthetic inputs shared by the CPU oracle and the HIP path.

This package holds workload shapes and random-number recipes only. It contains
none of the decoder's arithmetic: both the oracle and the HIP library receive
exactly the bytes produced here and compute independently from them.
"""
from .configs import DecoderConfig, Workload, WORKLOADS, TINY, LAYER_FULL, LAYER_SWA, FULL, LANE, param_count
from .gen import make_weights, make_prompt, make_kv, make_hidden, weight_names

__all__ = [
    "DecoderConfig", "Workload", "WORKLOADS", "TINY", "LAYER_FULL", "LAYER_SWA", "FULL", "LANE",
    "param_count", "make_weights", "make_prompt", "make_kv", "make_hidden", "weight_names",
]
