"""Seeded synthetic inputs for the NABLA hot path.

This package is shared by the CPU oracle's tests and by the HIP path's tests and
benchmark. It draws random numbers, smooths them into video-like fields and lays
tokens out in block order. It holds none of the method's arithmetic: no pooling,
no attention logits, no softmax, no selection.
"""

from .workloads import WORKLOADS, Workload, get_workload
from .generator import (
    block_order_permutation,
    make_field,
    make_inputs,
    make_dout,
    gaussian_taps,
    round_to_bf16,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "get_workload",
    "block_order_permutation",
    "make_field",
    "make_inputs",
    "make_dout",
    "gaussian_taps",
    "round_to_bf16",
]
