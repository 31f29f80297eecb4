"""CPU oracle of the biased-sigmoid top-4 MoE layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the HIP library never does.
"""

from .moe import *  # noqa: F401,F403
from .moe import (EXPERTS, FF, HIDDEN, ROUTED_SCALE, ROUTER_EPS, RMS_EPS,  # noqa: F401
                  TOP_K, Grouping, LayerResult, Routing)
