"""CPU oracle of the sparse MoE FFN layer (float64).  Test infrastructure only:
imported by the tests, the smoke check and the benchmark's CPU-baseline leg,
never by the HIP library or its Python binding."""
from .moe_oracle import *  # noqa: F401,F403
