"""Seeded synthetic inputs shared by the oracle's tests and the HIP path's tests and benchmark."""
from . import gen, configs  # noqa: F401
