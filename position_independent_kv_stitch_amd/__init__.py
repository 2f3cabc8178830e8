"""Position-independent KV-chunk stitching for MI355X (gfx950).

Relocates KV chunks cached at virtual offset 0 to arbitrary logical offsets
of a request: the rotary slice of every key is turned by the chunk's shift,
values and non-rotary dims are copied unchanged, and the first recompute_k
tokens of a chunk are left for a recompute pass.  All work runs in the HIP
library libpic_stitch.so (C ABI in include/pic_stitch.h); this package is
its thin binding.  Importing it loads the library and fails if it has not
been built.
"""
from ._binding import (EXPORTS, LIBRARY, PicError, Plan, Registry, attend,  # noqa: F401
                       attend_boundary, attend_latent, boundary_row_count,
                       load_library, match, match_records, rotate_inplace, rotate_paged,
                       rotate_workload, stitch, stream_copy)

load_library()
