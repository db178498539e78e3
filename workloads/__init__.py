"""Seeded synthetic decode workloads shared by the tests, the bench and the oracle.

This package only draws random inputs and writes down the order of pool
operations a workload performs (create / fork / append / free / attend / prefill).  It
holds none of the method's arithmetic: no slot computation, no block
allocation, no attention, no rounding to a low-precision type.  Both the
HIP path and the CPU oracle consume what it returns.
"""
from .configs import (  # noqa: F401
    Workload,
    CONFIG_NAMES,
    make_config,
    make_custom,
    make_prefill,
    make_prefill_config,
    PREFILL_NAMES,
)
