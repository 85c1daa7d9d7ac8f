"""Seeded synthetic workloads shaped like the DFlash 2 pages' benchmark setup.

Shared by the tests, ``bench.py`` and ``__graft_entry__.smoke()`` as the one
source of inputs for both the HIP library and the CPU oracle.  It computes
none of the five steps of the cycle: it draws random tensors and, where a
recipe asks for it, produces the inputs that other model components would
produce (the drafter's tap projection, the target model's logits) with
PyTorch's own matmul.
"""

from .configs import CONFIGS, Config, get_config
from .gen import make_cycle_inputs, make_generator

__all__ = ["CONFIGS", "Config", "get_config", "make_cycle_inputs", "make_generator"]
