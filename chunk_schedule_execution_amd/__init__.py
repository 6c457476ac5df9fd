"""MI355X-native executor for chunk-oriented collective schedules.

A chunk program (``dsl.Program``; library in ``programs``) is compiled by
``libccl.so`` into a plan -- dependency DAG, fused recv-reduce-copy-send
instructions, parallel instances on channels, sub-pipeline schedule, workgroup
allocation -- and one HIP kernel launch runs the whole collective over P virtual
ranks that share the GPU's HBM. ``capi`` is the ctypes binding of ``include/ccl.h``
under the same names; ``plan.Plan`` is a small object wrapper over it.

Importing this package loads ``lib/libccl.so`` and fails if it is not built.
"""

from . import capi  # noqa: F401  (loads libccl.so; raises ImportError if missing)
from .dsl import Buffer, ChunkRef, Program  # noqa: F401
from .plan import Plan, PlanConfig  # noqa: F401
from . import programs  # noqa: F401

__all__ = ["capi", "Buffer", "ChunkRef", "Program", "Plan", "PlanConfig", "programs"]
