"""oracle_top_kv_amd -- HySparse / HySparse2 attention hot path on MI355X (gfx950).

The compute lives in the HIP library ``libhysparse.so`` (C ABI in include/hysparse.h).  The
binding in ``oracle_top_kv_amd.hs`` only marshals torch tensors into pointers and sizes; it is
loaded lazily so that ``oracle_top_kv_amd.inputs`` can be used without the GPU library.
"""

__all__ = ["hs", "inputs"]


def __getattr__(name):
    if name == "hs":
        from . import hs as _hs
        return _hs
    if name == "inputs":
        from . import inputs as _inputs
        return _inputs
    raise AttributeError(name)
