"""Seeded synthetic inputs and the workload table, shared by the tests, the smoke
check and the benchmark. No attention arithmetic lives here."""
from .configs import ORDER, WORKLOADS, Workload, make_device, make_host, host_slice  # noqa: F401
