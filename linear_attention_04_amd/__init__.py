"""MI355X-native chunked KDA prefill: HIP kernels for gfx950 behind a C ABI.

Submodules are imported lazily so that ``linear_attention_04_amd.inputs`` can be
used without loading the HIP library.
"""
import importlib

__all__ = ["inputs", "kda"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
