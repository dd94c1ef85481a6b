"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark."""
from .gen import WORKLOADS, Workload, make_pool, make_queries, positions, acceptances, random_state  # noqa: F401
