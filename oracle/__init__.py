"""CPU oracle for the routed-expert MoE layer (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything here.  The GPU
library never routes through it and shares no code with it.
"""
from .moe_ref import *  # noqa: F401,F403
from .cache_ref import *  # noqa: F401,F403
from .rvq_ref import *  # noqa: F401,F403
