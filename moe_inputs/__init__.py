"""Seeded synthetic inputs shared by the fp64 oracle and the GPU path.

Holds data recipes only (shapes, random streams, storage rounding, stored row
tables); none of the layer's arithmetic lives here.
"""
from .configs import MoEConfig, NAMED, get  # noqa: F401
from . import generate, tables  # noqa: F401
