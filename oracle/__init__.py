"""CPU oracle for the MoE expert layer -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import anything in this package.  The GPU library never does.

Pinned functions (see ``tests/test_oracle_*.py``): routing, index builder,
permute/combine, expert forward, backward, FP8 codec and FP8 layer.  The
layer's output values have no worked example on the pages; they are pinned by
brute force, closed-form special cases and finite differences instead.
"""
from .moe_ref import *  # noqa: F401,F403
