"""Seeded synthetic inputs shared by the oracle side and the HIP side.

This package holds no arithmetic of the attention method: it draws random
numbers, rounds them to the storage type, and lays out block tables, slot
mappings and logical positions.  Both the tests' oracle runs and the GPU runs
consume the same arrays from here; neither side imports the other.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    make_workload,
    f32_to_bf16_bits,
    algorithmic_counts,
)
from .trace import RAG_TRACE, Trace, make_trace  # noqa: F401
