"""Seeded synthetic inputs shared by the tests, the bench and the oracle.

Input data only: nothing in this package computes any part of the method.
"""
from . import gen, workload  # noqa: F401
