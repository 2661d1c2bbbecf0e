"""MI355X-native chunked scan of a diagonal-decay selective state-space layer.

The compute path is the HIP library libssdscan (chunked_linear_recurrence_amd/csrc),
reached through a thin ctypes binding (``chunked_linear_recurrence_amd.ssd``).  Importing
this package does not load the library; the first call into the binding does, and fails
loudly when it is missing.
"""
from .workloads import WORKLOADS, Workload, ORDER, BENCH_WORKLOAD  # noqa: F401

__version__ = "0.1.0"
