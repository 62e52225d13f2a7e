"""Plain CPU oracle for the routed MoE expert-layer forward.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the test suite, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it, to
check and to time the HIP library.  It shares no code with that library.

What it computes is the plain result of an MoE layer, exactly as if every
expert were resident on the GPU: the pages state that offloaded experts are
neither simplified nor approximated and that the router is unchanged
(jansverre.net FreeToken article, section "Hva er FreeToken?").  The expert
cache therefore affects only where weights live, never the output; its state
is simulated separately in :mod:`oracle.cache`.

Floating point is fp64 except where the method fixes a precision: router
logits are rounded once to fp32, gates are stored as fp32, activations enter
as bf16 values.

Pins: every function here is checked by ``tests/test_oracle_*.py`` against
closed forms, library routines, independent formulations or brute force.
"""
from .mxfp4 import E2M1_VALUES, dequant, decode_e2m1  # noqa: F401
from .router import logits, topk, gates, route  # noqa: F401
from .dispatch import permutation  # noqa: F401
from .experts import expert_ffn, moe_layer  # noqa: F401
from .cache import SlotCache  # noqa: F401
from .mx import moe_layer_mx, quantize_mxfp8  # noqa: F401
