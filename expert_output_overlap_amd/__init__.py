"""MI355X-native MoE expert compute with tile-signalled return to owner ranks (HIP kernels behind a C ABI).

``binding`` exposes the C-ABI entry points of libmoe_overlap.so under their own names; ``runtime.MoePath`` holds
the device buffers of one problem.  Importing the package does not load the library; the first call does, and
raises if it has not been built.
"""
from . import binding  # noqa: F401

__all__ = ["binding"]
