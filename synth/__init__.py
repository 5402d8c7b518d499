"""Seeded synthetic inputs for the SmoothQuant W8A8 linear path (no method arithmetic)."""
from .workloads import WORKLOADS, Workload, get_workload, cast_to  # noqa: F401
