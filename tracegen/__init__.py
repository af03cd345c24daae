"""Seeded synthetic inputs (selection traces, KV rows, queries, workloads).

Input generation only; it holds none of the decode path's arithmetic.  Both
the HIP path's tests and benchmark and the CPU oracle take their inputs from
this package.
"""
from .values import kv_rows, q_block, kv_key, q_key, stream_key  # noqa: F401
from .trace import selection_trace, SelectionStream, growing_selection_trace, GrowingSelectionStream  # noqa: F401
from .workloads import Workload, make_workload, named_workload, NAMED, with_fp8, default_fp8_scales  # noqa: F401
