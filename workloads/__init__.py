"""Seeded synthetic workloads shared by the tests, the benchmark and the smoke
check.  This package draws inputs only: it holds none of the attention
method's arithmetic (no quantisation, no softmax, no tiling)."""
from .configs import CONFIGS, Config, get
from .gen import make_inputs, sample_rows

__all__ = ["CONFIGS", "Config", "get", "make_inputs", "sample_rows"]
