"""CPU oracle (float64, numpy) for the DLRM embedding-bag + interaction path.

TEST INFRASTRUCTURE ONLY: imported by tests/, by the package smoke check and by
the benchmark's CPU-baseline leg. The product path never imports it.
"""
from .dlrm_oracle import *  # noqa: F401,F403
from .dlrm_oracle import BagError, STATUS_BAD_INDEX, STATUS_BAD_OFFSETS  # noqa: F401
