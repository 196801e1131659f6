"""CPU oracle of the DeepSeekMoE layer forward (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It shares no code with the HIP library.
"""
from .oracle import *  # noqa: F401,F403
