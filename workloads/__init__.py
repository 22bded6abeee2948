"""Seeded synthetic inputs shared by the HIP path's tests/benchmark and the oracle.

This package holds input generation only -- none of the method's arithmetic.  Both the
oracle and the HIP library receive exactly the tensors produced here.
"""

from .configs import CONFIGS, WorkloadConfig, get_config
from .generate import MODE_CODES, controller_case, layer_inputs, moe_case, random_case

__all__ = ["CONFIGS", "WorkloadConfig", "get_config", "layer_inputs", "random_case", "controller_case", "moe_case", "MODE_CODES"]
