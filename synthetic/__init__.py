"""Seeded synthetic workloads (random draws and shapes only)."""
from .workloads import ModuleInput, Workload, small_case, workload, zipf_pmf  # noqa: F401
