"""MI355X-native engine for four-centre electron repulsion integrals.

The work happens in liberi_mi355x.so (HIP for gfx950, C ABI in include/eri.h);
this package is its thin Python binding.  PyTorch provides device memory and
streams only.
"""
from ._lib import (  # noqa: F401
    ERI_MAX_SIDE_STREAMS,
    ERI_NO_NORMALIZE,
    ERI_SPHERICAL,
    EriError,
    Plan,
    build_quartets,
    class_info,
    compute_batch,
    compute_deriv,
    compute_range,
    digest_J,
    digest_J_range,
    digest_JK,
    fp64_fma_tflops,
    load,
    strerror,
)
