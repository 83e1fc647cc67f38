"""Seeded synthetic inputs shared by the CPU oracle and the GPU path.

This package only draws numbers and lays out index arrays (context lengths,
block tables, which token rows each write covers). It holds none of the
method's arithmetic: no slot computation, no gather, no attention. Both the
oracle (``oracle/``) and the HIP path consume what it returns.
"""

from .gen import (CONFIGS, Workload, kv_bytes, make_custom, make_layers,  # noqa: F401
                  make_shared, make_tp_shard, make_workload, poison_pool)
from .engine import TokenRows, engine_requests  # noqa: F401
