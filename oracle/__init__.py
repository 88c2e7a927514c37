"""CPU oracle for MoE expert-parallel dispatch / combine -- test infrastructure
only (tests, the smoke check and the benchmark's CPU baseline use it; the
product library never does)."""
from .moe_oracle import *  # noqa: F401,F403
