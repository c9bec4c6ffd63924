"""Build-time generator of the per-class HIP kernels (never imported at run time)."""
