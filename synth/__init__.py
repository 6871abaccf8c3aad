"""Seeded synthetic workloads shared by the tests, the bench and the smoke check."""
from .workloads import HEADLINE, WORKLOADS, Workload  # noqa: F401
