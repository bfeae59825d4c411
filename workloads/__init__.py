"""Seeded synthetic inputs for the classifier-head loss workloads (see gen.py)."""
from .gen import WORKLOADS, Workload, make, workload, fp8_e4m3fn_values

__all__ = ["WORKLOADS", "Workload", "make", "workload", "fp8_e4m3fn_values"]
