"""Synthetic workloads (sizes and seeded input generators) shared by tests and bench."""
from .configs import WORKLOADS, Workload, workload, CANDS_16, CANDS_64, CANDS_128, CANDS_256, shape_code  # noqa: F401
