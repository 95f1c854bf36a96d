"""Seeded synthetic inputs for the speculative-sampling verification step.

This package is the only code shared by the fp64 oracle's tests and the HIP path's tests and
bench. It produces logits, draft tokens, uniforms and KV lengths, and holds none of the
verification arithmetic (no softmax, ratio, residual or inverse-CDF code): draft tokens are drawn
with the Gumbel-max trick, which samples softmax(l/T) without computing it. It also makes token
histories for prompt-lookup drafting (no matching code).
"""
from .bf16 import f32_to_bf16_bits, bf16_bits_to_f32
from .workloads import (CONFIGS, Workload, make_workload, make_tiny_random, config_by_name,
                        WORKLOAD_SEED_ROOT, as_greedy)
from .contexts import make_contexts, make_runs

__all__ = ["f32_to_bf16_bits", "bf16_bits_to_f32", "CONFIGS", "Workload", "make_workload",
           "make_tiny_random", "config_by_name", "WORKLOAD_SEED_ROOT", "make_contexts",
           "make_runs", "as_greedy"]
