"""Block top-k sparse-attention decode for MI355X (gfx950).

The compute path is libvx.so (hand-written HIP, C ABI in include/vx.h); this
package holds its ctypes binding, the step runtime and the seeded workload
generators. Importing the package does not load the library; the first call
into ``binding`` does, and fails loudly if it is missing.
"""

__all__ = ["binding", "step", "workloads", "build"]
