"""CPU oracle for the fused MLA query up-projection (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg import this
package. The product library never does, and shares no code with it.
"""
from .mla_oracle import *  # noqa: F401,F403
from .mla_oracle import (FMT_BSHD, FMT_SBHD, FMT_THD, Yarn, FwdResult, BwdResult)  # noqa: F401
