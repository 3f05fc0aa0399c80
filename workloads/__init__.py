"""Seeded synthetic inputs for the HSTU layer forward over a paged KV cache.

This module is shared by the tests, the benchmark and the smoke check.  It only
draws numbers and integer structure (lengths, page permutations, timestamps);
it holds none of the layer's arithmetic.  Both the fp64 oracle and the HIP
library receive exactly the arrays produced here.
"""
from .gen import (CONFIGS, TINY_FP32, B8_RECOMPUTE, B8_KV_HIT, B8_KV_HIT_LONG, B64_SERVING,  # noqa: F401
                  Workload, LayerInputs, make_workload, round_bf16)
