"""Seeded synthetic workloads (data only; no scoring arithmetic)."""
from .cases import Case, Shape, build_case, config_case, noise_ratio  # noqa: F401
