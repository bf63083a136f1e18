"""MI355X-native 2-D TM Maxwell FDTD propagator with an exact discrete adjoint.

``native`` binds the C ABI of ``libtm_fdtd.so`` (hand-written HIP kernels
for gfx950); ``inputs`` builds seeded synthetic workloads.
"""

from . import inputs  # noqa: F401

__all__ = ["inputs", "native", "build"]
