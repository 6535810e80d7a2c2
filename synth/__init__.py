"""Seeded synthetic workloads shared by the oracle's tests, the HIP path's tests and the benchmark."""
from .workloads import *  # noqa: F401,F403
from .prefill import *  # noqa: F401,F403
from .write import *  # noqa: F401,F403
