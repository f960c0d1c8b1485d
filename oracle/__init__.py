"""fp64 CPU oracle of the MS-GLA layer (test infrastructure only; never used by the GPU path)."""
from .msgla_oracle import *  # noqa: F401,F403
