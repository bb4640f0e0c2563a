"""Seeded synthetic inputs for the sparse decode step.

This package only draws random tensors and encodes them into the stored
formats the step consumes (bf16 bits, OCP e4m3fn bytes with a per-token scale,
4-bit channel codes and their bit planes, page tables, hot-buffer slot maps).
It holds none of the method's arithmetic -- no scores, no selection, no
attention, no read-depth allocation -- and it is shared by the tests, the
benchmark and the smoke check, which feed the same inputs to the HIP library
and to the CPU oracle.
"""
from .workloads import WORKLOADS, Workload, get  # noqa: F401
from .gen import (make_inputs, host_view, quantize_4bit, build_hot_buffer,  # noqa: F401
                  fixed_depths, random_depths, pinned_copy)
