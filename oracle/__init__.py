"""CPU oracle of the LaCT layer -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the bench's ``cpu_baseline`` leg
may import this package.  It shares no code with the HIP library and the
product path never calls it.
"""
from .lact import (  # noqa: F401
    NS_A, NS_B, NS_C, NS_EPS, NS_ITERS, apply, apply_head, dot_product_loss, gradient,
    layer, newton_schulz, norm_preserving_step, output_gate, rms_norm, shortconv2d, silu, sigmoid, stream,
    swiglu, update, update_head,
)
