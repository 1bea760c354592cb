"""CPU oracle for the MoE expert-FFN path.  TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 NumPy implementation of what the GPU path computes,
written from the pages' description of the method.  Only ``tests/``,
``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline`` leg may
import it; the product path never does.  It shares no code with the HIP
library and imports nothing from it.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import (SOFTMAX, SIGMOID, router_logits, biased_logits_f32, route, route_weights,
                         route_bwd,
                         rows_bound, permute, permute_bwd, gmm, tgmm, group_sum, swiglu, swiglu_bwd,
                         combine, combine_bwd, moe_forward, moe_backward)
from . import fp8_oracle as fp8  # noqa: F401
