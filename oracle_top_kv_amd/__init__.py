"""oracle_top_kv_amd -- HySparse / HySparse2 attention hot path on MI355X (gfx950).

The compute lives in the HIP library ``libhysparse.so`` (C ABI in include/hysparse.h).  The
binding in ``oracle_top_kv_amd.hs`` only marshals torch tensors into pointers and sizes; it is
imported lazily so that ``oracle_top_kv_amd.inputs`` can be used without the GPU library.
"""
import importlib

__all__ = ["hs", "inputs", "costs"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
