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


def __getattr__(name):
    # the fine-tuning reference needs torch; it is loaded on first use so that
    # processes that only encode and decode never import torch
    import importlib
    if name.startswith("__"):
        raise AttributeError(name)
    mod = importlib.import_module(__name__ + ".finetune_ref")
    try:
        return getattr(mod, name)
    except AttributeError:
        raise AttributeError("module 'oracle' has no attribute %r" % name) from None
