"""MI355X-native fused-dequantize Q4_K matrix-vector product.

The compute path is libq4k.so (hand-written HIP kernels for gfx950 behind a
C ABI, declared in include/q4k.h); `q4_packed_weight_amd.binding` is the thin
ctypes layer over it.  Nothing is imported eagerly so that the input
generators in `q4_packed_weight_amd.synth` can be used without loading the
GPU library.
"""

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
