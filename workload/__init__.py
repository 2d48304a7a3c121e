"""Seeded synthetic inputs shared by the CPU oracle (tests) and the HIP path.

Holds input descriptions and random draws only -- none of the MoE layer's
arithmetic lives here.
"""
from .configs import HEADLINE, WORKLOADS, Workload, custom, get  # noqa: F401
from . import generate  # noqa: F401
