"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the benchmark.

This package holds shapes, value distributions and seeds only. It contains none of the
method's arithmetic: no norm, quantizer, projection, convolution or recurrence.
"""
from .gen import (Dims, DIMS, WORKLOADS, LayerWeights, ProjWeights, layer_weights,
                  stack_weights, token_inputs, initial_states, bf16_round)

__all__ = ["Dims", "DIMS", "WORKLOADS", "LayerWeights", "ProjWeights", "layer_weights",
           "stack_weights", "token_inputs", "initial_states", "bf16_round"]
