"""MI355X-native mHC hot path: hc_pre / hc_post (forward and backward).

The compute runs in hand-written gfx950 HIP kernels behind the C ABI declared
in ``include/mhc.h`` (shared library ``libmhc.so`` built in-tree).  This
package only marshals arguments; import :mod:`residual_stream_amd.mhc` for the
binding.  Importing the package itself loads nothing.
"""

__all__ = ["inputs", "mhc"]
