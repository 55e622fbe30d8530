"""MI355X-native 8-bit block-wise optimizer step.

The compute path is the HIP library libbitopt.so (hand-written gfx950 kernels
behind a C ABI); `bit_optimizers_block_amd.bitopt` is its ctypes binding and
`bit_optimizers_block_amd.workloads` the seeded synthetic inputs of the benchmarks
and tests.
"""
__all__ = ["bitopt", "workloads"]
