"""Seeded synthetic inputs for the Hymba hybrid-head mixer.

This package draws random numbers and rounds them to the storage dtype; it
contains none of the mixer's arithmetic.  Both the fp64 oracle (through the
tests) and the GPU path (through the tests and the benchmark) take their
inputs from here, so the two sides see bit-identical values.
"""
from .configs import (WORKLOADS, LayerShape, Config, workload, TINY_F32, ABLATION_300M, SWA_8K, GLOBAL_8K,
                      DECODE_B128)
from .generate import (
    LayerParams, PrefillCase, DecodeCase,
    make_prefill_case, make_decode_case, make_layer_params, make_config_case,
    bf16_round, draw_normal,
)

__all__ = [
    "WORKLOADS", "LayerShape", "Config", "workload", "TINY_F32", "ABLATION_300M", "SWA_8K", "GLOBAL_8K",
    "DECODE_B128",
    "LayerParams", "PrefillCase", "DecodeCase",
    "make_prefill_case", "make_decode_case", "make_layer_params", "make_config_case",
    "bf16_round", "draw_normal",
]
