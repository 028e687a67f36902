"""MI355X-native sparse Mixture-of-Experts layer forward (HIP for gfx950).

The hot path runs in libmoe_mi355x.so (include/moe.h); ``api`` is its ctypes
binding (the library itself is loaded at the first call) and ``workloads``
holds the seeded synthetic inputs.
"""
from . import api, workloads  # noqa: F401

__all__ = ["api", "workloads"]
