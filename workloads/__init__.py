"""Seeded synthetic inputs shared by the tests, the oracle checks and the benchmark.

This package generates inputs only.  It computes no part of the verify rule:
no softmax, no acceptance test, no residual and no inverse-CDF sample.
"""
from .generators import *  # noqa: F401,F403
