"""Plain CPU oracle for the DeepSeekMoE feed-forward layer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it. It shares no code with the
HIP library (no kernels, headers, helpers or tables); the only thing both
sides see is the seeded input data.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_backward import *  # noqa: F401,F403
from .seq_balance import *  # noqa: F401,F403
from .fp8_backward import *  # noqa: F401,F403
