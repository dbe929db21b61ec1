"""Seeded synthetic workloads for the MiniMind FFN / top-k MoE forward and backward passes.

This package only *draws* inputs: shapes, seeds, distributions and storage
rounding.  It holds none of the method's arithmetic (no projection, softmax,
top-k or loss), so both the fp64 oracle and the HIP path can consume the same
bytes without sharing any computation.
"""
from .registry import WORKLOADS, Workload, get, intermediate_size
from .gen import (
    make_inputs,
    make_upstream,
    redraw_token_rows,
    to_f64,
    bf16_bits_from_f64,
    f64_from_bf16_bits,
)

__all__ = [
    "WORKLOADS",
    "Workload",
    "get",
    "intermediate_size",
    "make_inputs",
    "make_upstream",
    "redraw_token_rows",
    "to_f64",
    "bf16_bits_from_f64",
    "f64_from_bf16_bits",
]
