"""Block-sparse (Splash) attention forward for AMD MI355X (gfx950).

The work is done by ``libsplash.so`` (HIP kernels + host mask compiler,
C ABI in include/splash.h); this package only marshals arguments.  The
library is loaded on first use and its absence is an error.
"""

from .api import (MaskTables, bwd_tile, compile_mask, fwd_tile, fwd_tiles, splash_bwd, splash_fwd,
                  split_workspace_bytes)
from ._lib import SplashError

__all__ = ["MaskTables", "bwd_tile", "compile_mask", "fwd_tile", "fwd_tiles", "splash_bwd", "splash_fwd",
           "split_workspace_bytes", "SplashError"]
