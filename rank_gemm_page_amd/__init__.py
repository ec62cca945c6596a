"""Paged, heterogeneous-batch LoRA delta for MI355X (gfx950): HIP kernels behind a C ABI.

``slora`` is the ctypes binding of include/slora.h (same entry-point names);
``build`` compiles the library in tree; ``device_workload`` sets up seeded
synthetic workloads on the GPU through the binding.
"""
