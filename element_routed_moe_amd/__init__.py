"""MI355X (gfx950) implementation of one MatRIS-MoE interaction block.

The compute lives in ``libmlip.so`` (HIP kernels behind the C ABI of
``include/mlip.h``); ``element_routed_moe_amd.mlip`` is its Python binding and
``element_routed_moe_amd.synth`` draws the seeded synthetic workloads.
"""
__all__ = ["mlip", "synth", "build"]
