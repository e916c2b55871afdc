"""Seeded synthetic workloads (data only; no scoring arithmetic)."""
from .cases import Case, Shape, build_case, config_case, noise_ratio  # noqa: F401
from .paged import PagedPool, empty_pool, paged_from_case  # noqa: F401
