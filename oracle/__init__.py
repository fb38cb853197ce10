"""CPU oracle for the routed MoE FFN -- TEST INFRASTRUCTURE ONLY.

Plain, slow numpy evaluation of what the HIP library computes, used by the
tests, by the smoke check and by the CPU-baseline leg of the benchmark.  The
product path never imports it.  See ``oracle/moe_oracle.py`` and, for the
int8-activation variant, ``oracle/moe_oracle_q8.py``.
"""
from .moe_oracle import *  # noqa: F401,F403
