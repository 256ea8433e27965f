"""MI355X-native routed MoE block forward: routing, dispatch, grouped SwiGLU GEMM, combine.

The computation runs in hand-written HIP kernels for gfx950 behind the C-ABI
library ``libmoe.so`` (declared in ``include/moe.h``).  ``binding`` is a thin
ctypes layer over it; torch is used only for device memory and streams.
Importing this package does not load the library; ``binding.lib()`` does, and
raises if it has not been built.
"""
__all__ = ["binding", "workloads"]
