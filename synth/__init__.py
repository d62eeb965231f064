"""Seeded synthetic inputs for the MSA hot path (shared by tests, smoke and bench).

This package draws random numbers and lays out ragged document lengths. It holds
none of the method's arithmetic (no pooling, rotation, cosine, reduction,
selection or attention), so both the HIP path and the oracle may take inputs
from it without sharing any step of the computation.
"""
from .workloads import *  # noqa: F401,F403
