"""MS-GLA token-mixing layer forward for AMD MI355X (gfx950)."""
from .config import MsglaConfig, Workload, WORKLOADS, F32, BF16  # noqa: F401
