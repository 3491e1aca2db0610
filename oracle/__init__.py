"""CPU oracle for the MoE-layer forward and backward passes. Test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path (the HIP library and its
Python binding) never imports, calls or links it, and this package imports
nothing from the product path.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
from . import moe_backward  # noqa: F401
from .moe_backward import (layer_backward, routing_backward, expert_backward_sorted, dsilu,  # noqa: F401
                           token_backward, expert_grad_slices)
