"""CPU oracle for HyQuant-style hybrid-precision attention.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously-correct
reference that the HIP kernels are checked against. Only the test suite, the
smoke check in ``__graft_entry__`` and the benchmark's CPU-baseline leg may
import it; the product path (``kv_cache_amd``) never does, and it shares no
code with it.

Everything is numpy, accumulated in float64, one definition per step of the
method as the pages state it (see ``oracle/hyquant.py``). Decisions that turn
floating point into integers (quantisation codes) are taken in fp32, the
precision the kernels take them in, so that codes can be compared bit for
bit.
"""
from .hyquant import *  # noqa: F401,F403
