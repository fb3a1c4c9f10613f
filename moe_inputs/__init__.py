"""Seeded synthetic inputs and workload shapes of the gpt-oss-shaped MoE
layer.  Shared by the tests, the benchmark and the CPU oracle's harness; it
holds none of the layer's arithmetic (no product, routing or activation)."""
