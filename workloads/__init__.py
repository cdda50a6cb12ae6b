"""Seeded synthetic inputs for paged decode attention (shared by tests, bench and smoke).

This package only draws random numbers, encodes them into the stored formats and
places tokens into pages; it holds none of the attention arithmetic.
"""
from . import codec, layout, configs  # noqa: F401
from .configs import CONFIGS, Workload, Step  # noqa: F401
