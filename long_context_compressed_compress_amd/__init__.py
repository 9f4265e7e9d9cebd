"""CSA + HCA compressed attention for AMD MI355X (gfx950).

Submodules:
  libcsa     thin ctypes binding of the C-ABI library (include/libcsa.h); loads
             _native/libcsa.so and fails loudly if it is missing
  build      compiles the HIP kernels and the C-ABI into _native/libcsa.so
  workloads  seeded synthetic inputs of the five workloads
"""
