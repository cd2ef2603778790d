"""CPU oracle of the token-choice MoE FFN layer forward pass (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package. The product path never does: it runs on
the HIP library alone and fails loudly when that library is missing.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
