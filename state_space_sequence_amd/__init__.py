"""MI355X-native Mamba-3 SSM mixer core.

The compute path is a C-ABI shared library of hand-written HIP kernels for
gfx950 (``libm3.so``, declared in ``include/m3.h``). ``state_space_sequence_amd.m3``
is the thin Python binding over it (argument marshalling only); importing it
loads the library, and a missing library is an error, never a fallback.
``state_space_sequence_amd.inputs`` draws the seeded synthetic inputs.
"""
from . import inputs  # noqa: F401

__all__ = ["inputs"]
