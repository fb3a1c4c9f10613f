"""fp64 CPU oracles of the gpt-oss MoE MLP layer and of the attention steps
beside it -- TEST INFRASTRUCTURE.

Only the test suite, the package smoke check and the benchmark's CPU-baseline
leg may import this package.  The HIP product path never calls it.
"""
from . import attention_oracle, moe_oracle  # noqa: F401
