"""Seeded synthetic workload inputs (no layer arithmetic)."""
from .gen import *  # noqa: F401,F403
from .gen import WORKLOADS, Shape, Workload, ExpertWeights  # noqa: F401
