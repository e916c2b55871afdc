"""Seeded synthetic workloads (data only; no scoring arithmetic)."""
from .cases import (WORKLOAD_NAMES, Case, Shape, build_case, noise_ratio,  # noqa: F401
                    workload_case)
from .paged import PagedPool, empty_pool, paged_from_case  # noqa: F401
