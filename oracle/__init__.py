"""CPU oracle for the PT-DiT attention core (GIIM + TCM).

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, obviously-correct
float64 NumPy restatement of what the method computes. Only the tests, the
smoke check in __graft_entry__ and the CPU-baseline leg of bench.py may import
it. The GPU product path never imports, calls or links it, and it shares no
code with the GPU path (the seeded input generators in synth_inputs.py are the
only common module, and they hold none of the method's arithmetic).
"""
from .ptdit_oracle import *  # noqa: F401,F403
from .ptdit_backward import *  # noqa: F401,F403
from . import ptdit_backward as _bwd, ptdit_oracle as _fwd

__all__ = list(_fwd.__all__) + list(_bwd.__all__)
