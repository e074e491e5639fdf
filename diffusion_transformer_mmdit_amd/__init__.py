"""MI355X-native forward pass of the FLUX.2-style MMDiT denoiser.

The compute lives in the HIP library ``libflux.so`` (C ABI in ``include/flux.h``); this
package holds its sources (``csrc/``), the build script and a thin ctypes binding.
"""
from . import flux  # noqa: F401
from .flux import *  # noqa: F401,F403
