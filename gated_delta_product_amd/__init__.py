"""MI355X-native chunked Gated Delta Product (GDP) prefill forward.

The compute path is the C-ABI library ``libgdp.so`` (hand-written gfx950 HIP
kernels); :mod:`gated_delta_product_amd.binding` is a thin ctypes binding that
marshals torch tensors into it.  :mod:`gated_delta_product_amd.synth` draws
seeded synthetic inputs.
"""

__all__ = ["binding", "synth"]


def __getattr__(name):
    if name == "binding":
        from . import binding
        return binding
    if name == "synth":
        from . import synth
        return synth
    raise AttributeError(name)
