"""Paged KV cache for MI355X (gfx950): HIP kernels behind a C ABI (include/pa.h).

The Python names mirror the C ABI one to one (see ``_binding``).  Importing
fails if the library has not been built: there is no fallback path.
"""

from ._binding import *  # noqa: F401,F403
from ._binding import PAError, cache_desc, pa_cache_desc, LIB_PATH  # noqa: F401
