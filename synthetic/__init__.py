"""Seeded synthetic inputs shared by the oracle side and the HIP side."""
from . import gen  # noqa: F401
