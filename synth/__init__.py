"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle driver.

This package generates data only: key/value rows with a power-law spectrum,
decode queries, and the workload shapes they are drawn for. It holds none of
the compression method's arithmetic, so both the GPU path and the CPU oracle
can consume its output without sharing any of the method's code.
"""

from .configs import CONFIGS, Workload, get_config  # noqa: F401
from .gen import (  # noqa: F401
    bf16_round,
    haar_orthonormal,
    kv_rows,
    kv_rows_device,
    kv_rows_torch,
    queries,
    round_to,
    unit_key,
)
