"""MI355X-native chunked Gated Delta Product (GDP) prefill forward.

The compute path is the C-ABI library ``libgdp.so`` (hand-written gfx950 HIP
kernels); :mod:`gated_delta_product_amd.binding` is a thin ctypes binding that
marshals torch tensors into it.  :mod:`gated_delta_product_amd.synth` draws
seeded synthetic inputs.
"""
import importlib

__all__ = ["binding", "synth", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(__name__ + "." + name)
    raise AttributeError(name)
