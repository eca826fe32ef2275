"""Split-KV decode attention for AMD Instinct MI355X (gfx950).

The computation lives in ``libcrosscu.so`` (C ABI declared in
``include/crosscu.h``): a host planner that cuts the batch's KV tiles into one
equal chunk per compute unit, and persistent HIP kernels that stream the paged
KV cache and merge split sequences inside the same launch.

``binding``    ctypes marshalling of the C ABI (torch tensors -> raw pointers)
``workloads``  seeded synthetic decode workloads (inputs only)
``build``      compiles the library in-tree with hipcc for gfx950
"""
__all__ = ["binding", "workloads", "build"]
