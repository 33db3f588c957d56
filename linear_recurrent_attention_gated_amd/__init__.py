"""Gated-delta-rule (Gated DeltaNet) layer core for AMD Instinct MI355X (gfx950).

The compute lives in libgdn.so (C ABI: include/gdn.h, HIP kernels: csrc/); this
package holds its ctypes binding (``gdn``), the in-tree build (``build``) and the
seeded synthetic input generator (``inputs``).  Importing the package does not
load the library; the first call into ``gdn`` does, and fails loudly if it has
not been built.
"""
__all__ = ["gdn", "inputs", "build"]
