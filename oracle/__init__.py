"""CPU fp64 oracle for the LoopVQ hot path -- TEST INFRASTRUCTURE ONLY.

Only the tests, the package smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path (the HIP library and its binding)
never calls it and shares no code with it.

Every function is the plain definition from the LoopVQ review (arXiv
2611.05304), written in NumPy float64, with no blocking or fusion.
"""
from .loopvq_ref import *  # noqa: F401,F403
from .tasq_perm import *  # noqa: F401,F403,E402
from .kmeans_ref import *  # noqa: F401,F403,E402
from .finetune_ref import *  # noqa: F401,F403,E402
