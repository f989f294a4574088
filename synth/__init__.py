"""Seeded synthetic inputs shared by the oracle, the GPU tests and the benchmark."""
from . import inputs
