"""Seeded synthetic workloads for the sigmoid-routed MoE layer.

Shared by the CPU oracle (tests only) and the HIP path's tests and
benchmark. Holds configs and random draws only, none of the layer's
arithmetic.
"""
from . import configs, gen  # noqa: F401
from .configs import MoEConfig, ALL, get  # noqa: F401
