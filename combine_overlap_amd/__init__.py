"""MI355X (gfx950) library for one expert-parallel rank's MoE-layer share with
tile-signalled combine overlap.

The compute path is the HIP library libmoe_overlap.so (C ABI in
include/moe_overlap.h); `ops` is its thin Python binding and `share.MoEShare`
owns the device buffers of one shape. There is no non-GPU fallback.
"""
from . import _abi  # noqa: F401
from ._abi import (MOE_CONSUMER_AUTO, MOE_GATE_SIGMOID, MOE_GATE_SOFTMAX,  # noqa: F401
                   MOE_MODE_OVERLAP, MOE_MODE_ROLE_SWITCH, MOE_MODE_SEQUENTIAL, MoeError)

__all__ = ["ops", "share", "MoeError", "MOE_MODE_OVERLAP", "MOE_MODE_SEQUENTIAL", "MOE_MODE_ROLE_SWITCH",
           "MOE_CONSUMER_AUTO", "MOE_GATE_SOFTMAX", "MOE_GATE_SIGMOID"]
