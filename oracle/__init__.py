"""fp64 CPU oracle for position-independent KV stitching.

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are its only users.  The product path never
imports it, and it shares no code with the HIP library.
"""
from .ref import (attend, attend_boundary, attend_latent, boundary_rows, inv_freq,  # noqa: F401
                  recompute_ranges, rotate_inplace, rotate_paged, validate_rotate_paged,
                  round_bf16,
                  stitch, validate_inplace, validate_stitch)
