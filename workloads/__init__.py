"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the benchmark.

This module only draws random numbers and lays them out as arrays.  It holds
none of the integral arithmetic (no normalisation, no Gaussian products, no
screening): both the CPU oracle and the HIP library receive exactly these raw
arrays and do their own work on them.
"""
from .configs import (  # noqa: F401
    ShellSet,
    Workload,
    CONFIG_SEEDS,
    make_config,
    class_batch,
    cluster,
    random_psd_density,
    subset_shells,
)
