"""CPU oracle of the W4A16 MoE layer. Test infrastructure only (tests/, smoke(), bench cpu_baseline)."""
from .oracle import *  # noqa: F401,F403
from .router import route  # noqa: F401
