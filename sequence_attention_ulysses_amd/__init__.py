"""MI355X-native Ulysses sequence-parallel exchange (P ranks emulated as P slabs of one GPU).

The work runs in ``libuly.so`` (hand-written gfx950 HIP kernels behind the C ABI
of ``include/uly.h``); this package is its thin binding.
"""
from .api import (UlyssesContext, describe, height_split, rope_table_1d,  # noqa: F401
                  rope_table_3d)
from ._lib import (UlyBroken, UlyCacheFull, UlyDtypeError, UlyError, UlyHipError,  # noqa: F401
                   UlyInvalidArgument, UlyNotFound, UlyOverlap, UlyUnsupported)

MODE_SCATTER = 0
MODE_GATHER = 1
