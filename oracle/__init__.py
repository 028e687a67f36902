"""CPU oracle of the MoE-layer forward: test infrastructure only.

Only the test-suite, the entry file's smoke check and the benchmark's CPU
baseline may import this package; the HIP library never does.
"""
from . import moe_oracle  # noqa: F401
