"""MI355X-native MoE expert hot path: router, top-K, 4/2-bit groupwise-affine
dequantised GEMV with fused SwiGLU, down projection and gated combine.

The compute runs in the HIP library `libmoe.so` (C ABI, see include/moe.h);
`bit_dequant_expert_route_amd.moe` is a thin ctypes binding over it.  The
binding is imported lazily so that host-only tools (the input generator) do not
need the library.
"""
import importlib

__all__ = ["moe", "synth"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
