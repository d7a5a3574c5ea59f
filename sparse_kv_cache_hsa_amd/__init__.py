"""MI355X-native RocketKV decode path: SnapKV++ eviction and Hybrid Sparse
Attention in hand-written HIP kernels (librkv), with a thin ctypes binding.

Submodules are imported on demand: ``rkv`` (the binding; loads librkv),
``synth`` (seeded synthetic inputs), ``workloads`` (the benchmark
configurations) and ``build`` (compiles librkv).
"""
__all__ = ["rkv", "synth", "workloads", "build"]
