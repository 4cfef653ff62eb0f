"""MI355X-native Mamba-3 SSM mixer core.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libm3.so``, declared in ``include/m3.h``). ``state_space_sequence_amd.m3``
is the thin Python binding over it (argument marshalling only); the library is
loaded on first use and its absence is an error, never a fallback.
"""
from . import inputs  # noqa: F401  (seeded synthetic inputs; no method arithmetic)

__all__ = ["inputs", "m3"]


def __getattr__(name):
    if name == "m3":
        from . import m3 as _m3
        return _m3
    raise AttributeError(name)
